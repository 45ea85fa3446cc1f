// Chunkwise forward of Kimi Delta Attention (KDA) on gfx950.
//
// The recurrence (per batch b, head h; state S is dk x dv, fp32):
//   S_t = (I - beta_t k_t k_t^T) Diag(e^{g_t}) S_{t-1} + beta_t k_t v_t^T,
//   o_t = S_t^T q_t,   g_t clamped to [-5, 0],
// is evaluated 16 tokens at a time. Unrolling it over a chunk with entering
// state S0 (r, s index tokens of the chunk, Gamma_r the inclusive per-channel
// sum of g up to r, gamma = Gamma_16):
//   Qt = e^Gamma Q,  Kt = e^Gamma K,  Kh = e^-Gamma K,  Kb = e^(gamma - Gamma) K
//   A  = strictly_lower(diag(beta) Kt Kh^T),   M = lower_incl(Qt Kh^T)
//   Tm = (I + A)^-1,   W = Tm diag(beta) Kt,   Ut = Tm diag(beta) V
//   U  = Ut - W S0,    O = Qt S0 + M U,        S_16 = Diag(e^gamma) S0 + Kb^T U
// Only the last line couples chunks. The -5 floor keeps e^-Gamma <= e^80 over
// 16 tokens, inside bf16 range, so the diagonal (intra-chunk) products run as
// dense matrix-core tiles with no position-by-position path ("K3 tech report"
// podcast transcript, the exchange on the decay bound; "Kimi K3 goes
// trillion-scale with sparse MoE efficiency" subtitles, cue 14).
//
// Two kernels:
//  kda_chunk_prep   one wavefront per (b, h, chunk), all chunks in parallel:
//                   decay scan with DPP row scans (a 16-lane row = the 16
//                   tokens of a chunk), scaled operands, Gram tiles A and M on
//                   the matrix cores, (I + A)^-1 by forward substitution in
//                   LDS, W on the matrix cores; writes one workspace record
//                   per chunk in matrix-core fragment order.
//  kda_state_pass   one wavefront per (b, h, 16-column slice of dv): keeps its
//                   dk x 16 slice of S in registers for the whole sequence and
//                   applies the last two lines chunk after chunk. Columns of S
//                   never interact, so slices need no communication.
//
// Lane conventions (l = lane, c16 = l % 16, gq = l / 16): a 16x16 MFMA output
// tile has lane l holding rows 4*gq + i (i = 0..3) of column c16. In the prep
// kernel lane l owns token c16 and key channels 16*m + 4*gq + i of it; the
// contraction slots of every dk-contraction are mapped to channels so that the
// state slice, held in output layout, is directly the B operand of W S and
// Qt S (no shuffles on the sequential path).
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename InT>
struct Path {
  static constexpr bool kF32 = std::is_same<InT, float>::value;
  // element type of the state-pass matrix operands
  using Op = typename std::conditional<kF32, float, _Float16>::type;
};

// ---------------------------------------------------------------------------
// Record fragment addressing (see RecordLayout). Each lane's values come in
// groups of 4 consecutive rows/tokens i = 0..3.
//   W, Q: value (m, i) = X[token c16][channel 16m + 4gq + i]
//   Kb:   value (m, i) = Kb[token 4gq + i][channel 16m + c16]
//   M:    value i      = M[c16][4gq + i]
//   Tb:   value i      = Tm[c16][4gq + i] * beta_{4gq + i}
//   eg:   e^gamma[channel 16m + 4gq + i] at float index gq*dk/4 + 4m + i
// fp16 path: W, Q packed per pair of tiles (2p, 2p+1) as 8 halves (16 B) at
// ((p*64 + l) * 16); Kb as 4 halves at ((m*64 + l) * 8); M as hi then lo
// halves (l*8 and 512 + l*8); Tb at l*8.
// fp32 path: W, Q as 4 floats at ((m*64 + l) * 16); Kb likewise; M, Tb at l*16.
// ---------------------------------------------------------------------------

template <typename InT, int DK, int GATE>
__global__ __launch_bounds__(64) void kda_chunk_prep(const InT* __restrict__ q,
                                                     const InT* __restrict__ k,
                                                     const InT* __restrict__ g,
                                                     const InT* __restrict__ beta,
                                                     uint8_t* __restrict__ ws, int64_t T,
                                                     int64_t H, int64_t NC, RecordLayout L) {
  constexpr bool F32 = Path<InT>::kF32;
  constexpr int NM = DK / 16;
  constexpr int LDK = DK + 4;  // padded LDS row (conflict-free transposed reads)
  using Op = typename Path<InT>::Op;
  // Kt and Kb are staged in the state-pass operand type (fp16 for bf16
  // inputs: both are rounded to it on use anyway), which keeps the LDS of
  // this one-wave workgroup small enough for 4 waves per SIMD.
  __shared__ float s_beta[16];
  __shared__ Op s_kt[16 * LDK];
  __shared__ Op s_kb[16 * LDK];
  __shared__ float s_A[16][17];
  __shared__ float s_T[16][17];

  const int l = threadIdx.x, c16 = l & 15, gq = l >> 4;
  const int64_t wg = blockIdx.x;  // ((b * NC) + n) * H + h
  const int64_t h = wg % H;
  const int64_t bn = wg / H;
  const int64_t n = bn % NC;
  const int64_t b = bn / NC;
  const int64_t t = n * 16 + c16;
  const bool valid = t < T;
  const size_t tok = static_cast<size_t>((b * T + (valid ? t : 0)) * H + h);

  uint8_t* rec = ws + static_cast<size_t>((b * H + h) * NC + n) * L.bytes;

  // ---- load this lane's token: 4*NM channels of q, k, g, kept packed ----
  // (converted where used, so the whole chunk's fp32 operands are never live
  // at once; bf16 inputs take 2 VGPRs per 4 channels)
  using Raw = typename std::conditional<F32, float4, uint2>::type;
  Raw rq[NM], rk[NM], rg[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const size_t off = tok * DK + 16 * m + 4 * gq;
    if (valid) {
      rq[m] = *reinterpret_cast<const Raw*>(q + off);
      rk[m] = *reinterpret_cast<const Raw*>(k + off);
      rg[m] = *reinterpret_cast<const Raw*>(g + off);
    } else {
      rq[m] = rk[m] = rg[m] = Raw{};
    }
  }
  if (gq == 0) s_beta[c16] = valid ? load_in(beta, tok) : 0.f;

  // ---- per pair of 16-channel groups: decay scan, scaled operands, Gram ----
  // Channel (m, i) = 16m + 4gq + i. The Gram contraction over the 8 channels
  // of pair p takes slot j = 4(m - 2p) + i (any bijection serves a Gram
  // product); the same slots order the Qt record (state-pass layout).
  // MrawT = Kh Qt^T is M^T: its output layout puts M[c16][4gq + i] in this
  // lane, the layout the record wants, with no transpose through LDS.
  f32x4 Araw = zero4(), MrawT = zero4();
#pragma unroll
  for (int p = 0; p < NM / 2; ++p) {
    float qt[8], kt[8], kh[8], eg[8];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int m = 2 * p + jj;
      float xq[4], xk[4], xg[4];
      unpack4(rq[m], xq);
      unpack4(rk[m], xk);
      unpack4(rg[m], xg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // padded tokens past T carry log-decay 0 whatever the gate
        const float x = (valid ? gate_decay<GATE>(xg[i]) : 0.f) * kLog2e;
        const float G = row_inclusive_prefix_sum(x);    // log2 e^Gamma_r
        const float Gb = row_exclusive_suffix_sum(x);   // log2 e^(gamma - Gamma_r)
        // the -5 floor bounds |G|, |Gb| by 80 log2(e) over 16 tokens, so every
        // power of two here is a normal float: the hardware exp2 needs no
        // range reduction
        const float E = __builtin_amdgcn_exp2f(G);
        const float Eh = __builtin_amdgcn_exp2f(-G);
        const float Eb = __builtin_amdgcn_exp2f(Gb);
        const int j = 4 * jj + i;
        qt[j] = E * xq[i];
        kt[j] = E * xk[i];
        kh[j] = Eh * xk[i];
        eg[j] = E;
        s_kt[c16 * LDK + 16 * m + 4 * gq + i] = static_cast<Op>(kt[j]);
        s_kb[c16 * LDK + 16 * m + 4 * gq + i] = static_cast<Op>(Eb * xk[i]);
      }
    }
    if constexpr (F32) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        Araw = mma_16x16x4_f32(kt[j], kh[j], Araw);
        MrawT = mma_16x16x4_f32(kh[j], qt[j], MrawT);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const size_t off = static_cast<size_t>((2 * p + jj) * 64 + l) * 16;
        *reinterpret_cast<float4*>(rec + L.q + off) =
            make_float4(qt[4 * jj], qt[4 * jj + 1], qt[4 * jj + 2], qt[4 * jj + 3]);
      }
    } else {
      // bf16 operands carry the e^{+-Gamma} range; each is split into a bf16
      // high part and a bf16 remainder (hi*hi + hi*lo + lo*hi) for accuracy.
      bf16x8 kt_hi, kt_lo, kh_hi, kh_lo, qt_hi, qt_lo;
      f16x8 qv;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        kt_hi[j] = static_cast<__bf16>(kt[j]);
        kt_lo[j] = static_cast<__bf16>(kt[j] - static_cast<float>(kt_hi[j]));
        kh_hi[j] = static_cast<__bf16>(kh[j]);
        kh_lo[j] = static_cast<__bf16>(kh[j] - static_cast<float>(kh_hi[j]));
        qt_hi[j] = static_cast<__bf16>(qt[j]);
        qt_lo[j] = static_cast<__bf16>(qt[j] - static_cast<float>(qt_hi[j]));
        qv[j] = static_cast<Op>(qt[j]);
      }
      Araw = mma_16x16x32_bf16(kt_hi, kh_hi, Araw);
      Araw = mma_16x16x32_bf16(kt_hi, kh_lo, Araw);
      Araw = mma_16x16x32_bf16(kt_lo, kh_hi, Araw);
      MrawT = mma_16x16x32_bf16(kh_hi, qt_hi, MrawT);
      MrawT = mma_16x16x32_bf16(kh_lo, qt_hi, MrawT);
      MrawT = mma_16x16x32_bf16(kh_hi, qt_lo, MrawT);
      *reinterpret_cast<f16x8*>(rec + L.q + static_cast<size_t>(p * 64 + l) * 16) = qv;
    }
    if (c16 == 15) {  // e^gamma for this lane's channels of the pair
      float* egp = reinterpret_cast<float*>(rec + L.eg) + gq * (DK / 4) + 8 * p;
      *reinterpret_cast<float4*>(egp) = make_float4(eg[0], eg[1], eg[2], eg[3]);
      *reinterpret_cast<float4*>(egp + 4) = make_float4(eg[4], eg[5], eg[6], eg[7]);
    }
  }
  __syncthreads();  // s_beta, s_kt, s_kb visible

  // ---- mask: A strictly lower with row scale beta_r ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * gq + i, s = c16;
    s_A[r][s] = (s < r) ? s_beta[r] * Araw[i] : 0.f;
  }
  __syncthreads();

  // ---- Tm = (I + A)^-1, column c16 per lane, by forward substitution ----
  // Tm[r][j] = delta_rj - sum_{s<r} A[r][s] Tm[s][j] (A strictly lower).
  {
    float tc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == c16) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) acc -= s_A[r][s] * tc[s];
      tc[r] = acc;
    }
    if (gq == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_T[r][c16] = tc[r];
    }
  }
  __syncthreads();

  // tb[i] = Tm[c16][s] beta_s and mf[i] = M[c16][s] (M lower incl. diag)
  // for s = 4gq + i: this lane's fragments of the record
  float tb[4], mf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 4 * gq + i;
    tb[i] = s_T[c16][s] * s_beta[s];
    mf[i] = (s <= c16) ? MrawT[i] : 0.f;
  }

  // ---- W^T tiles = Kt^T (diag(beta) Tm^T): lane gets W[c16][16m+4gq+i] ----
  float w[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    Op a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = s_kt[(4 * gq + i) * LDK + 16 * m + c16];
    f32x4 acc = zero4();
    if constexpr (F32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = mma_16x16x4_f32(a[i], tb[i], acc);
    } else {
      f16x4 av, bv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = a[i];
        bv[i] = static_cast<_Float16>(tb[i]);
      }
      acc = mma_16x16x16_f16(av, bv, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) w[m][i] = acc[i];
  }

  // ---- write the rest of the record ----
  if constexpr (F32) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const size_t off = static_cast<size_t>(m * 64 + l) * 16;
      *reinterpret_cast<float4*>(rec + L.w + off) = make_float4(-w[m][0], -w[m][1], -w[m][2], -w[m][3]);
      float kb4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kb4[i] = s_kb[(4 * gq + i) * LDK + 16 * m + c16];
      *reinterpret_cast<float4*>(rec + L.kbar + off) = make_float4(kb4[0], kb4[1], kb4[2], kb4[3]);
    }
    *reinterpret_cast<float4*>(rec + L.m + l * 16) = make_float4(mf[0], mf[1], mf[2], mf[3]);
    *reinterpret_cast<float4*>(rec + L.tb + l * 16) = make_float4(tb[0], tb[1], tb[2], tb[3]);
  } else {
#pragma unroll
    for (int p = 0; p < NM / 2; ++p) {
      f16x8 wv;
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = static_cast<Op>(-w[2 * p + (j >> 2)][j & 3]);
      *reinterpret_cast<f16x8*>(rec + L.w + static_cast<size_t>(p * 64 + l) * 16) = wv;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      f16x4 kv;
#pragma unroll
      for (int i = 0; i < 4; ++i) kv[i] = s_kb[(4 * gq + i) * LDK + 16 * m + c16];
      *reinterpret_cast<f16x4*>(rec + L.kbar + static_cast<size_t>(m * 64 + l) * 8) = kv;
    }
    f16x4 mh, ml, tv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mh[i] = static_cast<Op>(mf[i]);
      ml[i] = static_cast<Op>(mf[i] - static_cast<float>(mh[i]));
      tv[i] = static_cast<Op>(tb[i]);
    }
    *reinterpret_cast<f16x4*>(rec + L.m + l * 8) = mh;
    *reinterpret_cast<f16x4*>(rec + L.m + 512 + l * 8) = ml;
    *reinterpret_cast<f16x4*>(rec + L.tb + l * 8) = tv;
  }
}

// ---------------------------------------------------------------------------
// Sequential state pass.
// ---------------------------------------------------------------------------

template <typename InT, int DK>
struct ChunkFrags {
  static constexpr bool F32 = Path<InT>::kF32;
  static constexpr int NM = DK / 16;
  // W and Q: fp16 -> NM/2 x 8 halves; fp32 -> NM x 4 floats (same values)
  typename std::conditional<F32, f32x4, f16x8>::type w[F32 ? NM : NM / 2];
  typename std::conditional<F32, f32x4, f16x8>::type q[F32 ? NM : NM / 2];
  typename std::conditional<F32, f32x4, f16x4>::type kb[NM];
  typename std::conditional<F32, f32x4, f16x4>::type mh, ml, tb;
  f32x4 eg[NM];
  float vv[4];

  // Record fragments of one chunk; `rec` is uniform across the wavefront, so
  // every access is a scalar base plus a 32-bit per-lane byte offset.
  __device__ __forceinline__ void load_record(const uint8_t* rec, const RecordLayout& L, int l,
                                              int gq) {
    const uint8_t* rw = rec + L.w;
    const uint8_t* rq = rec + L.q;
    const uint8_t* rk = rec + L.kbar;
    const uint8_t* rm = rec + L.m;
    const uint8_t* rt = rec + L.tb;
    const uint8_t* re = rec + L.eg;
    if constexpr (F32) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint32_t off = static_cast<uint32_t>(m * 64 + l) * 16;
        w[m] = ld_at<f32x4>(rw, off);
        q[m] = ld_at<f32x4>(rq, off);
        kb[m] = ld_at<f32x4>(rk, off);
      }
      mh = ld_at<f32x4>(rm, static_cast<uint32_t>(l) * 16);
      tb = ld_at<f32x4>(rt, static_cast<uint32_t>(l) * 16);
    } else {
#pragma unroll
      for (int p = 0; p < NM / 2; ++p) {
        const uint32_t off = static_cast<uint32_t>(p * 64 + l) * 16;
        w[p] = ld_at<f16x8>(rw, off);
        q[p] = ld_at<f16x8>(rq, off);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) kb[m] = ld_at<f16x4>(rk, static_cast<uint32_t>(m * 64 + l) * 8);
      mh = ld_at<f16x4>(rm, static_cast<uint32_t>(l) * 8);
      ml = ld_at<f16x4>(rm, 512u + static_cast<uint32_t>(l) * 8);
      tb = ld_at<f16x4>(rt, static_cast<uint32_t>(l) * 8);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) eg[m] = ld_at<f32x4>(re, static_cast<uint32_t>(gq * NM + m) * 16);
  }

  // V rows 4gq + i of a chunk; `vchunk` (uniform) points at the chunk's first
  // token of this (b, h), vb[i] = ((4gq + i) * H * DV + col) * sizeof(InT)
  // (byte offsets). Tokens at or past `valid` (a last partial chunk) read as
  // zero.
  __device__ __forceinline__ void load_v(const InT* vchunk, const uint32_t vb[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = ld_in_at(vchunk, vb[i]);
  }
  __device__ __forceinline__ void load_v_partial(const InT* vchunk, const uint32_t vb[4], int gq,
                                                 int valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = (4 * gq + i < valid) ? ld_in_at(vchunk, vb[i]) : 0.f;
  }
};

// One chunk of the sequential pass on the fp16-operand path, with the
// chunk's V rows 4gq + i (column c16) given in fp16. With kOT the output comes
// back transposed: O^T = S^T Qt^T + U^T M^T is the same pair of products with
// the operands swapped (each fragment already holds what the other operand
// position needs), and it leaves lane (c16, gq) with token c16's value
// columns 4gq .. 4gq+3, one contiguous vector store.
template <bool kOT, typename InT, int DK>
__device__ __forceinline__ f32x4 chunk_step_h(const ChunkFrags<InT, DK>& cur, f16x4 v16,
                                              f32x4 (&S)[DK / 16]) {
  constexpr int NM = DK / 16;
  f32x4 U, O;
  // Every accumulation chain below uses one MFMA shape (16x16x32). Two shapes
  // chained through an accumulator need wait states on gfx950 that the
  // compiler does not insert; the 16-deep token contractions are issued as
  // 16x16x32 with the upper 16 slots zero (or, for M U, holding the
  // low-order part of M against a second copy of U). K=16 and K=32 issue at
  // the same rate on gfx950, so the padding costs nothing.
  f16x8 tbz, vz;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tbz[i] = cur.tb[i];
    tbz[i + 4] = static_cast<_Float16>(0.f);
    vz[i] = v16[i];
    vz[i + 4] = static_cast<_Float16>(0.f);
  }
  U = mma_16x16x32_f16(tbz, vz, zero4());                                    // Ut = Tb V
  f16x8 sh[NM / 2];
#pragma unroll
  for (int p = 0; p < NM / 2; ++p)
#pragma unroll
    for (int j = 0; j < 8; ++j) sh[p][j] = static_cast<_Float16>(S[2 * p + (j >> 2)][j & 3]);
  O = zero4();
#pragma unroll
  for (int p = 0; p < NM / 2; ++p) {
    U = mma_16x16x32_f16(cur.w[p], sh[p], U);                                // U = Ut - W S
    O = kOT ? mma_16x16x32_f16(sh[p], cur.q[p], O)                           // O^T = S^T Qt^T
            : mma_16x16x32_f16(cur.q[p], sh[p], O);                          // O = Qt S
  }
  f16x8 uu, mhl;
  f16x4 u4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 x = static_cast<_Float16>(U[i]);
    uu[i] = x;
    uu[i + 4] = x;
    u4[i] = x;
    mhl[i] = cur.mh[i];
    mhl[i + 4] = cur.ml[i];
  }
  O = kOT ? mma_16x16x32_f16(uu, mhl, O)                                     // O^T += U^T M^T
          : mma_16x16x32_f16(mhl, uu, O);                                    // O += (Mhi + Mlo) U
  // S = Diag(e^gamma) S + Kb^T U: the accumulator input is the VALU product
  // S * e^gamma, never another MFMA's output, so the 16x16x16 shape is safe.
#pragma unroll
  for (int m = 0; m < NM; ++m) S[m] = mma_16x16x16_f16(cur.kb[m], u4, S[m] * cur.eg[m]);
  return O;
}

// One chunk of the sequential pass on a dk x 16 state slice S (output layout):
// U = Tb V - W S,  O = Qt S + M U,  S <- Diag(e^gamma) S + Kb^T U.  Returns O.
template <typename InT, int DK>
__device__ __forceinline__ f32x4 chunk_step(const ChunkFrags<InT, DK>& cur, f32x4 (&S)[DK / 16]) {
  constexpr int NM = DK / 16;
  f32x4 U, O;
  if constexpr (Path<InT>::kF32) {
    U = zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i) U = mma_16x16x4_f32(cur.tb[i], cur.vv[i], U);   // Ut = Tb V
    O = zero4();
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        U = mma_16x16x4_f32(cur.w[m][i], S[m][i], U);                        // U = Ut - W S
        O = mma_16x16x4_f32(cur.q[m][i], S[m][i], O);                        // O = Qt S
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) O = mma_16x16x4_f32(cur.mh[i], U[i], O);      // O += M U
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      S[m] = S[m] * cur.eg[m];
#pragma unroll
      for (int i = 0; i < 4; ++i) S[m] = mma_16x16x4_f32(cur.kb[m][i], U[i], S[m]);
    }
  } else {
    f16x4 v16;
#pragma unroll
    for (int i = 0; i < 4; ++i) v16[i] = static_cast<_Float16>(cur.vv[i]);
    O = chunk_step_h<false>(cur, v16, S);
  }
  return O;
}

template <typename InT, typename OutT, int DK>
__global__ __launch_bounds__(64) void kda_state_pass(const InT* __restrict__ v,
                                                     const uint8_t* __restrict__ ws,
                                                     const float* S0, OutT* __restrict__ o,
                                                     float* ST, float* __restrict__ snap,
                                                     int64_t snap_chunks, int64_t T, int64_t H,
                                                     int64_t DV, int64_t NC, int64_t nslices,
                                                     int64_t nheads, RecordLayout L) {
  constexpr bool F32 = Path<InT>::kF32;
  constexpr int NM = DK / 16;
  using Frags = ChunkFrags<InT, DK>;
  const int l = threadIdx.x, c16 = l & 15, gq = l >> 4;

  // XCD-aware numbering: workgroups are dealt round-robin to the 8 XCDs, so
  // all slices of one head get ids congruent mod 8 and share an XCD's L2
  // for the head's workspace records.
  const int64_t wgid = blockIdx.x;
  const int64_t xcd = wgid & 7, kk = wgid >> 3;
  const int64_t head = xcd + 8 * (kk / nslices);
  const int64_t slice = kk % nslices;
  if (head >= nheads) return;
  const int64_t b = head / H, h = head % H;
  const int64_t col = slice * 16 + c16;

  // state slice: S[m][i] = S[16m + 4gq + i][col]
  f32x4 S[NM];
  const size_t sbase = static_cast<size_t>(head) * DK * DV + col;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[m][i] = S0 ? S0[sbase + static_cast<size_t>(16 * m + 4 * gq + i) * DV] : 0.f;

  // Uniform per-(b,h) bases; per-lane offsets fixed for the whole sequence.
  const uint8_t* rec0 = ws + static_cast<size_t>(head) * NC * L.bytes;
  const size_t hb = static_cast<size_t>(b * T * H + h) * DV;   // token 0 of (b, h)
  const InT* vb = v + hb;
  OutT* ob = o + hb;
  const size_t chunk_elems = static_cast<size_t>(16 * H) * DV;
  // per-lane byte offsets of rows 4gq + i of a chunk (H * DV <= 2^25, so
  // 16 * H * DV elements of at most 4 bytes fit in 32 bits)
  uint32_t vbo[4], obo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t e = static_cast<uint32_t>((4 * gq + i) * H * DV + col);
    vbo[i] = e * static_cast<uint32_t>(sizeof(InT));
    obo[i] = e * static_cast<uint32_t>(sizeof(OutT));
  }

  const int64_t NF = T / 16;  // full chunks
  // Full chunks: records prefetched two chunks ahead (fp32 path: one) into
  // fragment buffers whose roles rotate by unrolling (a register copy between
  // buffers would force a wait for the loads in flight); the last full chunk
  // is re-read past the end instead of branching around the load.
  auto fetch = [&](Frags& f, int64_t c) __attribute__((always_inline)) {
    c = c < NF - 1 ? c : NF - 1;
    f.load_record(rec0 + static_cast<size_t>(c) * L.bytes, L, l, gq);
    f.load_v(vb + static_cast<size_t>(c) * chunk_elems, vbo);
  };
  // Snapshots (snap_chunks > 0): the state after every snap_chunks full
  // chunks, i.e. after tokens [0, (j+1) * 16 * snap_chunks), goes to snapshot
  // j, laid out [B, T / (16 * snap_chunks), H, DK, DV]. Only full chunks can
  // end one. With snap_chunks = 0 the per-chunk test is never true; the
  // uniform branch stays in the loop either way, because this compiler then
  // keeps the record prefetch in flight across iterations (without it, it
  // drains every load at the loop head: 2.8 ms instead of 2.2 ms at 64K
  // tokens x 32 heads).
  int64_t next_snap = snap_chunks;
  float* snap_b = nullptr;
  if (snap_chunks > 0) {
    const int64_t ns = NF / snap_chunks;
    snap_b = snap + (static_cast<size_t>(b * ns) * H + h) * DK * DV + col;
  }
  auto finish = [&](int64_t n, f32x4 O) __attribute__((always_inline)) {
    OutT* oc = ob + static_cast<size_t>(n) * chunk_elems;
#pragma unroll
    for (int i = 0; i < 4; ++i) st_out_at(oc, obo[i], O[i]);
    if (n + 1 == next_snap) {
      float* sp = snap_b + static_cast<size_t>(n / snap_chunks) * H * DK * DV;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[static_cast<size_t>(16 * m + 4 * gq + i) * DV] = S[m][i];
      next_snap += snap_chunks;
    }
  };
  if (NF > 0) {
    Frags f0, f1, f2;
    if constexpr (F32) {
      fetch(f0, 0);
      for (int64_t n = 0; n < NF; n += 2) {
        fetch(f1, n + 1);
        finish(n, chunk_step(f0, S));
        if (n + 1 >= NF) break;
        fetch(f0, n + 2);
        finish(n + 1, chunk_step(f1, S));
      }
    } else {
      fetch(f0, 0);
      fetch(f1, 1);
      for (int64_t n = 0; n < NF; n += 3) {
        fetch(f2, n + 2);
        finish(n, chunk_step(f0, S));
        if (n + 1 >= NF) break;
        fetch(f0, n + 3);
        finish(n + 1, chunk_step(f1, S));
        if (n + 2 >= NF) break;
        fetch(f1, n + 4);
        finish(n + 2, chunk_step(f2, S));
      }
    }
  }
  if (NC > NF) {  // last partial chunk: padded tokens read as zero and are not stored
    const int valid = static_cast<int>(T - NF * 16);
    Frags f;
    f.load_record(rec0 + static_cast<size_t>(NF) * L.bytes, L, l, gq);
    f.load_v_partial(vb + static_cast<size_t>(NF) * chunk_elems, vbo, gq, valid);
    const f32x4 O = chunk_step(f, S);
    OutT* oc = ob + static_cast<size_t>(NF) * chunk_elems;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * gq + i < valid) st_out_at(oc, obo[i], O[i]);
  }
  if (ST) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) ST[sbase + static_cast<size_t>(16 * m + 4 * gq + i) * DV] = S[m][i];
  }
}

// ---------------------------------------------------------------------------
// Sequential state pass, fp16-operand path: a loader wave and a compute wave.
//
// The sequential chain (U = Ut - W S, S <- Diag(e^gamma) S + Kb^T U) runs on
// one wavefront per (b, h, 16-column slice). Fed from global memory directly,
// that wavefront waits on its own prefetch loads: the compiler's wait
// placement in an unrolled prefetch loop leaves only about one chunk of
// loads in flight, and HBM latency then sets the pace. Here a second
// wavefront of the same workgroup streams each chunk's record and V tile
// from HBM into a ring of LDS slots, several chunks ahead, with coalesced
// 16-byte loads (and converts V to fp16, transposed for the MFMA operand);
// the compute wavefront only reads LDS. One LDS-only barrier per chunk keeps
// the two in step. Barrier 0 follows the loader's prologue, barrier n + 1
// ends the compute wave's step n:
//   prologue         the loader fills slots 0 .. kRing-2 with chunks
//                    0 .. kRing-2;
//   compute step n   uses chunk n (read into registers during step n - 1)
//                    and reads chunk n + 1 from its slot;
//   loader step n    between barriers n and n + 1, writes chunk n + kRing - 1
//                    into slot (n - 1) % kRing, whose previous chunk the
//                    compute wave finished reading before barrier n - 1;
//                    the write is complete at barrier n + 1, and the chunk is
//                    read after barrier n + kRing - 3 >= n + 1.
// The loader keeps kStages chunks of loads in registers, so each chunk's
// loads are issued kStages steps before they are written to LDS. Measured
// settings: kStages = 4 with kRing = 4 (2 stages: 2.06 ms; 6 slots slower;
// taking the barrier before the LDS writes instead of after: 3% slower).
// ---------------------------------------------------------------------------

constexpr int kRing = 4;
constexpr int kStages = 4;
static_assert(kRing >= 3, "the compute wave reads one slot ahead of the one it uses");


// LDS-only release/acquire around a workgroup barrier: orders this wave's LDS
// accesses against the other wave's, without waiting for global loads.
// The scheduling barriers keep the instruction scheduler from moving work
// across steps (it would otherwise hoist the loader's use of loaded data to
// the top of the loop, where it must wait for every load in flight).
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

// 16-byte record loads per lane at dk = 128, plus one V load: the loads of
// kStages - 1 chunks stay in flight at each commit, and that count must fit
// the 6-bit load counter the waits encode.
constexpr int kRingLoadsPerChunk = 14 + 1;
static_assert((kStages - 1) * kRingLoadsPerChunk <= 63, "loads in flight exceed the wait counter");

template <int DK>
struct RingGeom {
  static constexpr int kRec = DK == 128 ? 14336 : 8192;  // record bytes (bf16 inputs)
  static constexpr int kUnits = kRec / 1024;             // 16-byte loads per lane
  static constexpr int kSlot = kRec + 512;               // + V^T tile, 16x16 fp16
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DK>
struct LoaderStage {
  u32x4 r[RingGeom<DK>::kUnits];
  u32x2 v;
  bool v_ok;  // the V token exists (applied at commit: a select right after
              // the load would make the compiler wait for it there)
};

template <typename OutT, int DK>
__global__ __launch_bounds__(128) void kda_state_pass_ring(const uint16_t* __restrict__ v,
                                                           const uint8_t* __restrict__ ws,
                                                           const float* S0, OutT* __restrict__ o,
                                                           float* ST, float* __restrict__ snap,
                                                           int64_t snap_chunks, int64_t T, int64_t H,
                                                           int64_t DV, int64_t NC, int64_t nslices,
                                                           int64_t nheads, RecordLayout L) {
  using G = RingGeom<DK>;
  constexpr int NM = DK / 16;
  using Frags = ChunkFrags<uint16_t, DK>;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * G::kSlot];

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, c16 = l & 15, gq = l >> 4;
  // XCD-aware numbering, as in kda_state_pass.
  const int64_t wgid = blockIdx.x;
  const int64_t xcd = wgid & 7, kk = wgid >> 3;
  const int64_t head = xcd + 8 * (kk / nslices);
  const int64_t slice = kk % nslices;
  if (head >= nheads) return;  // whole workgroup
  const int64_t b = head / H, h = head % H;
  const uint8_t* rec0 = ws + static_cast<size_t>(head) * NC * G::kRec;
  const size_t hb = static_cast<size_t>(b * T * H + h) * DV;
  const size_t chunk_elems = static_cast<size_t>(16 * H) * DV;
  const int64_t NF = T / 16;
  const int64_t NCS = (NC + kStages - 1) / kStages * kStages;  // loader steps (and barriers)

  if (wave == 0) {
    // ---------------- loader ----------------
    // V: lane -> token tv of the chunk, columns cv .. cv+3 of the slice.
    const int tv = l >> 2, cv = 4 * (l & 3);
    const uint32_t vcol = static_cast<uint32_t>(slice * 16 + cv);
    const uint32_t vrow = static_cast<uint32_t>(H * DV);  // elements per token
    const uint16_t* vb = v + hb;
    // Loads are unconditional (chunks past the end re-read the last one, V
    // tokens past T are zeroed by a select): a branch around them would make
    // the compiler's wait counting conservative at the join.
    auto issue = [&](LoaderStage<DK>& st, int64_t c) __attribute__((always_inline)) {
      const int64_t cc = c < NC ? c : NC - 1;
      const uint8_t* src = rec0 + static_cast<size_t>(cc) * G::kRec;
#pragma unroll
      for (int j = 0; j < G::kUnits; ++j) st.r[j] = ld_at<u32x4>(src, static_cast<uint32_t>(j * 64 + l) * 16);
      // tokens past T (last partial chunk) read the last token instead: every
      // load stays inside v; the value is zeroed at commit
      const int64_t tmax = T - 1 - cc * 16;
      const uint32_t t = static_cast<uint32_t>(tv < tmax ? tv : tmax);
      st.v = ld_at<u32x2>(vb + static_cast<size_t>(cc) * chunk_elems, (t * vrow + vcol) * 2u);
      st.v_ok = c * 16 + tv < T;
    };
    // Commits are unconditional too: a chunk past the end lands in a slot
    // the compute wave reads no more (the same reuse distance as in the
    // steady state), and is never read.
    auto commit = [&](const LoaderStage<DK>& st, int64_t c) __attribute__((always_inline)) {
      {
        uint8_t* dst = ring + static_cast<int>(c % kRing) * G::kSlot;
#pragma unroll
        for (int j = 0; j < G::kUnits; ++j) st_at<u32x4>(dst, static_cast<uint32_t>(j * 64 + l) * 16, st.r[j]);
        // V^T[col][token] in fp16: the compute lane (c16, gq) reads the four
        // tokens 4gq .. 4gq+3 of column c16 as one 8-byte word.
        const uint32_t v0 = st.v_ok ? st.v[0] : 0u, v1 = st.v_ok ? st.v[1] : 0u;
        const float x[4] = {__uint_as_float(v0 << 16), __uint_as_float(v0 & 0xffff0000u),
                            __uint_as_float(v1 << 16), __uint_as_float(v1 & 0xffff0000u)};
        _Float16* vt = reinterpret_cast<_Float16*>(dst + G::kRec);
#pragma unroll
        for (int i = 0; i < 4; ++i) vt[(cv + i) * 16 + tv] = static_cast<_Float16>(x[i]);
      }
    };
    LoaderStage<DK> st[kStages];
    // prologue: chunks 0 .. kStages-1 in flight, then slots 0 .. kRing-2
    // filled (each commit refills its stage kStages chunks ahead)
#pragma unroll
    for (int c = 0; c < kStages; ++c) issue(st[c], c);
#pragma unroll
    for (int c = 0; c < kRing - 1; ++c) {
      commit(st[c % kStages], c);
      issue(st[c % kStages], c + kStages);
    }
    ring_barrier();
    // step n writes chunk n + kRing - 1 (slot (n - 1) % kRing) from its
    // stage and refills that stage with the chunk kStages further on. The
    // loop runs a multiple of kStages steps with no exit in between (an exit
    // inside would make the compiler drain every load at the loop's back
    // edge); the compute wave pads its barriers to the same count.
    for (int64_t n = 0; n < NCS; n += kStages) {
#pragma unroll
      for (int k = 0; k < kStages; ++k) {
        const int64_t c = n + k + kRing - 1;
        commit(st[(k + kRing - 1) % kStages], c);
        issue(st[(k + kRing - 1) % kStages], c + kStages);
        ring_barrier();
      }
    }
    return;
  }

  // ---------------- compute ----------------
  const int64_t col = slice * 16 + c16;
  f32x4 S[NM];
  const size_t sbase = static_cast<size_t>(head) * DK * DV + col;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[m][i] = S0 ? S0[sbase + static_cast<size_t>(16 * m + 4 * gq + i) * DV] : 0.f;
  OutT* ob = o + hb;
  // output in transposed fragments: lane (c16, gq) holds token c16, value
  // columns slice*16 + 4gq .. +3 of the chunk
  const uint32_t obt =
      static_cast<uint32_t>(c16 * H * DV + slice * 16 + 4 * gq) * static_cast<uint32_t>(sizeof(OutT));
  int64_t next_snap = snap_chunks;
  float* snap_b = nullptr;
  if (snap_chunks > 0) {
    const int64_t ns = NF / snap_chunks;
    snap_b = snap + (static_cast<size_t>(b * ns) * H + h) * DK * DV + col;
  }
  auto finish = [&](int64_t n, f32x4 OT) __attribute__((always_inline)) {
    st_out4_at(ob + static_cast<size_t>(n) * chunk_elems, obt, OT);
    if (n + 1 == next_snap) {
      float* sp = snap_b + static_cast<size_t>(n / snap_chunks) * H * DK * DV;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[static_cast<size_t>(16 * m + 4 * gq + i) * DV] = S[m][i];
      next_snap += snap_chunks;
    }
  };
  auto read = [&](Frags& f, f16x4& vh, int64_t c) __attribute__((always_inline)) {
    const uint8_t* src = ring + static_cast<int>(c % kRing) * G::kSlot;
    f.load_record(src, L, l, gq);
    vh = ld_at<f16x4>(src + G::kRec, static_cast<uint32_t>(c16 * 16 + 4 * gq) * 2);
  };
  ring_barrier();
  Frags f0, f1;
  f16x4 v0, v1;
  read(f0, v0, 0);
  // Full chunks, two per iteration (the fragment buffers alternate by
  // position, never by copy); the next chunk's slot is read one step ahead.
  int64_t n = 0;
  for (; n + 1 < NF; n += 2) {
    read(f1, v1, n + 1);
    finish(n, chunk_step_h<true>(f0, v0, S));
    ring_barrier();
    if (n + 2 < NC) read(f0, v0, n + 2);
    finish(n + 1, chunk_step_h<true>(f1, v1, S));
    ring_barrier();
  }
  if (n < NF) {  // an odd last full chunk, in f0
    if (n + 1 < NC) read(f1, v1, n + 1);
    finish(n, chunk_step_h<true>(f0, v0, S));
    ring_barrier();
    ++n;
    if (NC > NF) {  // then the partial chunk, in f1
      const int valid = static_cast<int>(T - NF * 16);
      const f32x4 OT = chunk_step_h<true>(f1, v1, S);
      if (c16 < valid) st_out4_at(ob + static_cast<size_t>(NF) * chunk_elems, obt, OT);
      ring_barrier();
    }
  } else if (NC > NF) {  // even number of full chunks: the partial chunk is in f0
    const int valid = static_cast<int>(T - NF * 16);
    const f32x4 OT = chunk_step_h<true>(f0, v0, S);
    if (c16 < valid) st_out4_at(ob + static_cast<size_t>(NF) * chunk_elems, obt, OT);
    ring_barrier();
  }
  for (int64_t k = NC; k < NCS; ++k) ring_barrier();  // match the loader's steps
  if (ST) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) ST[sbase + static_cast<size_t>(16 * m + 4 * gq + i) * DV] = S[m][i];
  }
}

// T = 0: the final state is the initial one (or zeros).
__global__ void kda_copy_state(const float* S0, float* ST, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) ST[i] = S0 ? S0[i] : 0.f;
}

template <typename InT, int DK, int GATE>
hipError_t launch_prep_typed(const ChunkFwdArgs& a, hipStream_t stream) {
  const RecordLayout L = record_layout(DK, Path<InT>::kF32);
  const int64_t NC = (a.T + 15) / 16;
  const int64_t blocks = a.B * NC * a.H;
  hipLaunchKernelGGL((kda_chunk_prep<InT, DK, GATE>), dim3(static_cast<uint32_t>(blocks)), dim3(64), 0,
                     stream, static_cast<const InT*>(a.q), static_cast<const InT*>(a.k),
                     static_cast<const InT*>(a.g), static_cast<const InT*>(a.beta),
                     static_cast<uint8_t*>(a.workspace), a.T, a.H, NC, L);
  return hipGetLastError();
}

// Snapshots are taken only when at least one falls inside the sequence.
inline bool wants_snapshots(const ChunkFwdArgs& a) {
  return a.snapshots != nullptr && a.snapshot_every > 0 && a.T >= a.snapshot_every;
}

template <typename InT, typename OutT, int DK>
hipError_t launch_pass_typed(const ChunkFwdArgs& a, hipStream_t stream) {
  const int64_t nslices = a.dv / 16;
  const RecordLayout L = record_layout(DK, Path<InT>::kF32);
  const int64_t NC = (a.T + 15) / 16;
  const int64_t nheads = a.B * a.H;
  const int64_t blocks = 8 * nslices * ((nheads + 7) / 8);
  const int64_t snap_chunks = wants_snapshots(a) ? a.snapshot_every / 16 : 0;
  if constexpr (!Path<InT>::kF32) {
    if (L.bytes != RingGeom<DK>::kRec) return hipErrorInvalidValue;  // layout and ring disagree
    hipLaunchKernelGGL((kda_state_pass_ring<OutT, DK>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(128), 0, stream, static_cast<const uint16_t*>(a.v),
                       static_cast<const uint8_t*>(a.workspace), a.S0, static_cast<OutT*>(a.o),
                       a.S_T, snap_chunks > 0 ? a.snapshots : nullptr, snap_chunks, a.T, a.H, a.dv,
                       NC, nslices, nheads, L);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((kda_state_pass<InT, OutT, DK>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(64), 0, stream, static_cast<const InT*>(a.v),
                     static_cast<const uint8_t*>(a.workspace), a.S0, static_cast<OutT*>(a.o),
                     a.S_T, snap_chunks > 0 ? a.snapshots : nullptr, snap_chunks, a.T, a.H, a.dv, NC,
                     nslices, nheads, L);
  return hipGetLastError();
}

template <typename InT, int DK>
hipError_t launch_prep_gate(const ChunkFwdArgs& a, hipStream_t s) {
  return a.gate == kGateSigmoid ? launch_prep_typed<InT, DK, kGateSigmoid>(a, s)
                                : launch_prep_typed<InT, DK, kGateLogDecay>(a, s);
}

template <typename InT>
hipError_t launch_prep_dk(const ChunkFwdArgs& a, hipStream_t s) {
  return a.dk == 64 ? launch_prep_gate<InT, 64>(a, s) : launch_prep_gate<InT, 128>(a, s);
}

template <typename InT, typename OutT>
hipError_t launch_pass_dk(const ChunkFwdArgs& a, hipStream_t s) {
  return a.dk == 64 ? launch_pass_typed<InT, OutT, 64>(a, s) : launch_pass_typed<InT, OutT, 128>(a, s);
}

// T = 0: S_T is S0 (or zeros) unless it is S0 itself.
hipError_t launch_empty(const ChunkFwdArgs& a, hipStream_t stream) {
  if (a.S_T && a.S_T != a.S0) {
    const int64_t n = a.B * a.H * a.dk * a.dv;
    hipLaunchKernelGGL(kda_copy_state, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0,
                       stream, a.S0, a.S_T, n);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_chunk_prep(const ChunkFwdArgs& a, hipStream_t stream) {
  if (a.B * a.H == 0 || a.T == 0) return hipSuccess;
  return a.in_dtype == 0 ? launch_prep_dk<float>(a, stream) : launch_prep_dk<uint16_t>(a, stream);
}

hipError_t launch_chunk_state_pass(const ChunkFwdArgs& a, hipStream_t stream) {
  if (a.B * a.H == 0) return hipSuccess;
  if (a.T == 0) return launch_empty(a, stream);
  const bool in32 = a.in_dtype == 0, out32 = a.out_dtype == 0;
  if (in32) return out32 ? launch_pass_dk<float, float>(a, stream) : launch_pass_dk<float, uint16_t>(a, stream);
  return out32 ? launch_pass_dk<uint16_t, float>(a, stream) : launch_pass_dk<uint16_t, uint16_t>(a, stream);
}

hipError_t launch_chunk_fwd(const ChunkFwdArgs& a, hipStream_t stream) {
  const hipError_t e = launch_chunk_prep(a, stream);
  if (e != hipSuccess) return e;
  return launch_chunk_state_pass(a, stream);
}

}  // namespace kda
