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
// Two phases, each a kernel:
//  prep         all chunks in parallel: decay scan with a DPP row scan (a
//               16-lane row = the 16 tokens of a chunk) and a row broadcast of
//               its last token for e^gamma, scaled operands, Gram
//               tiles A and M on the matrix cores, (I + A)^-1 by forward
//               substitution in LDS, W on the matrix cores; writes workspace
//               records in matrix-core fragment order.
//  state pass   one workgroup per (b, h, 16-column slice of dv): keeps its
//               dk x 16 slice of S in registers for the whole sequence and
//               applies the lines that couple chunks, in order. Columns of S
//               never interact, so slices need no communication.
// fp32 inputs use fp32 matrix cores, one record per chunk (kda_chunk_prep,
// kda_state_pass). bf16 inputs use fp16 operands for the state products (v
// stays exact in bf16 products), one record per pair of chunks, and the state
// pass advances 32 tokens per step (kda_chunk_prep_pair,
// kda_state_pass_ring32).
//
// Lane conventions (l = lane, c16 = l % 16, gq = l / 16): a 16x16 MFMA output
// tile has lane l holding rows 4*gq + i (i = 0..3) of column c16. In the prep
// kernels lane l owns token c16 (key channels 16*m + 4*gq + i of it in the
// fp32 prep, 32*p + 8*gq + i in the pair prep); the records' contraction slots
// of every dk-contraction are mapped to channels 16*m + 4*gq + i, so that the
// state slice, held in output layout, is directly the B operand of W S and
// Qt S (no shuffles on the sequential path).
#include <mutex>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename InT>
constexpr bool kIsF32 = std::is_same<InT, float>::value;

// What a state pass computes: kPassOutputs, the forward (o, S_T);
// kPassState, only the final state; kPassTransition, the state transition of
// the tokens (each 16-column slice starts from its columns of the dk x dk
// identity with v = 0, so S_T is the matrix F with S_out = F S_in + the
// state reached from S_in = 0); kPassFE, F and that state E in one pass over
// dk + dv columns (bf16 inputs). The last three write no outputs.
constexpr int kPassOutputs = 0, kPassState = 1, kPassTransition = 2, kPassFE = 3;

// Four fp32 values as bf16 [high parts | low parts]: x = hi + lo to about 16
// bits. A 16-deep contraction against an exact bf16 operand repeated in both
// halves then costs one 32-deep matrix-core product.
__device__ __forceinline__ bf16x8 split_bf16(const float (&x)[4]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = static_cast<__bf16>(x[i]);
    r[i + 4] = static_cast<__bf16>(x[i] - static_cast<float>(r[i]));
  }
  return r;
}

// Eight bf16 values in 16 bytes, and their fp32 values. The type's alignment
// is the inputs' documented 8 bytes; the hardware serves a 16-byte vector load
// from any dword-aligned address.
typedef uint32_t u32x4a8 __attribute__((ext_vector_type(4), aligned(8)));
__device__ __forceinline__ void unpack8(const u32x4a8& x, float out[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    out[2 * d] = __uint_as_float(x[d] << 16);
    out[2 * d + 1] = __uint_as_float(x[d] & 0xffff0000u);
  }
}

// ---------------------------------------------------------------------------
// Record fragment addressing. Each lane's values come in groups of 4
// consecutive rows/tokens i = 0..3.
//   W, Q: value (m, i) = X[token c16][channel 16m + 4gq + i]
//   Kb:   value (m, i) = Kb[token 4gq + i][channel 16m + c16]
//   M:    value i      = M[c16][4gq + i]
//   Tb:   value i      = Tm[c16][4gq + i] * beta_{4gq + i}
//   eg:   e^gamma[channel 16m + 4gq + i] at float index gq*dk/4 + 4m + i
// Per-chunk record (fp32 inputs, RecordLayout): W, Q, Kb as 4 floats at
// ((m*64 + l) * 16); M, Tb at l*16.
// Pair record (bf16 inputs, PairLayout): W, Q packed per pair of tiles
// (2p, 2p+1) as 8 fp16 halves (16 B) at ((p*64 + l) * 16); Kb of both chunks
// as 8 halves at ((m*64 + l) * 16), chunk 1 in the low four; the M tiles as 8
// halves at l*16 (two tiles side by side, or a high and a low part); Tb of
// each chunk as 8 bf16 at l*16 (high parts, then low parts); -C21 as 4 halves
// at l*8.
// ---------------------------------------------------------------------------

// Chunk prep for fp32 inputs: one wavefront per (b, h, chunk), fp32 matrix
// cores throughout; writes the per-chunk record.
template <int DK, int GATE>
__global__ __launch_bounds__(64) void kda_chunk_prep(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ g,
                                                     const float* __restrict__ beta,
                                                     uint8_t* __restrict__ ws, int64_t T,
                                                     int64_t H, int64_t NC, RecordLayout L) {
  constexpr int NM = DK / 16;
  constexpr int LDK = DK + 4;  // padded LDS row (conflict-free transposed reads)
  __shared__ float s_beta[16];
  __shared__ float s_kt[16 * LDK];
  __shared__ float s_kb[16 * LDK];
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

  // ---- load this lane's token: 4*NM channels of q, k, g ----
  using Raw = float4;
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
        // the -5 floor bounds |G| by 80 log2(e) over 16 tokens, so every power
        // of two here is a normal float: the hardware exp2 needs no range
        // reduction
        const float E = __builtin_amdgcn_exp2f(G);
        const float Eh = __builtin_amdgcn_exp2f(-G);
        const float Eg = row_broadcast_last(E);  // e^gamma, the decay to the chunk's end
        const int j = 4 * jj + i;
        qt[j] = E * xq[i];
        kt[j] = E * xk[i];
        kh[j] = Eh * xk[i];
        eg[j] = E;
        s_kt[c16 * LDK + 16 * m + 4 * gq + i] = kt[j];
        s_kb[c16 * LDK + 16 * m + 4 * gq + i] = kh[j] * Eg;  // e^(gamma - Gamma_r) k
      }
    }
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
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = s_kt[(4 * gq + i) * LDK + 16 * m + c16];
    f32x4 acc = zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mma_16x16x4_f32(a[i], tb[i], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[m][i] = acc[i];
  }

  // ---- write the rest of the record ----
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
}

// ---------------------------------------------------------------------------
// Pair prep (bf16 inputs): the record for two consecutive chunks c1 = 2s and
// c2 = 2s + 1, so that the state pass can advance 32 tokens per step. With
// S0 the state entering c1, S1 = Diag(e^g1) S0 + Kb1^T U1 the state entering
// c2 (g1 = gamma of c1, per channel), the two chunks' lines become
//   U1 = Ut1 - W1 S0
//   U2 = Ut2 - W2 Diag(e^g1) S0 - C21 U1,          C21 = W2 Kb1^T
//   O1 = Qt1 S0 + M1 U1
//   O2 = Qt2 Diag(e^g1) S0 + M21 U1 + M2 U2,       M21 = Qt2 Kb1^T
//   S2 = Diag(e^(g1 + g2)) S0 + [Diag(e^g2) Kb1^T | Kb2^T] [U1; U2]
// (the off-diagonal 16-token tiles, C21 and M21, are dense products as well).
// Every factor is a product of retentions, so nothing here exceeds 1 in size.
// One wavefront per chunk (the per-chunk work is that of kda_chunk_prep);
// wavefront 1 also forms C21 and M21 from wavefront 0's Kb1 through LDS.
// ---------------------------------------------------------------------------

template <int DK, int GATE>
__global__ __launch_bounds__(128) void kda_chunk_prep_pair(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ g,
                                                           const uint16_t* __restrict__ beta,
                                                           uint8_t* __restrict__ ws, int64_t T,
                                                           int64_t H, int64_t NPR, PairLayout L) {
  constexpr int NM = DK / 16;
  constexpr int LDK = DK + 8;  // padded LDS row: 16-byte aligned, conflict-free transposed reads
  using Op = _Float16;
  __shared__ float s_beta[2][16];
  __shared__ __attribute__((aligned(16))) Op s_kt[2][16 * LDK];
  __shared__ __attribute__((aligned(16))) Op s_kb[2][16 * LDK];
  __shared__ __attribute__((aligned(16))) Op s_qt[2][16 * LDK];  // Qt of each chunk (before the e^g1 factor)
  __shared__ float s_eg[2][DK];       // e^gamma of each chunk, per channel
  __shared__ float s_A[2][16][17];
  __shared__ float s_T[2][16][17];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c16 = l & 15, gq = l >> 4;
  const int64_t wg = blockIdx.x;  // ((b * NPR) + s) * H + h
  const int64_t h = wg % H;
  const int64_t bs = wg / H;
  const int64_t sp = bs % NPR;
  const int64_t b = bs / NPR;
  const int64_t n = 2 * sp + w;  // this wavefront's chunk
  const int64_t t = n * 16 + c16;
  const bool valid = t < T;
  const size_t tok = static_cast<size_t>((b * T + (valid ? t : 0)) * H + h);
  uint8_t* rec = ws + static_cast<size_t>((b * H + h) * NPR + sp) * L.bytes;

  // ---- loads, kept packed until used: 8 consecutive channels per lane ----
  // Every lane loads (tokens past T read token 0 of the sequence) and the
  // padding tokens are zeroed where each value is first used: loads complete
  // in order, and a use right after the loads (beta's conversion, or zeros
  // written over a pending load) would wait for all of them before the
  // channel loop starts.
  const uint16_t braw = beta[tok];
  u32x4a8 rq[NM / 2], rk[NM / 2], rg[NM / 2];
#pragma unroll
  for (int p = 0; p < NM / 2; ++p) {
    const size_t off = tok * DK + 32 * p + 8 * gq;
    rq[p] = *reinterpret_cast<const u32x4a8*>(q + off);
    rk[p] = *reinterpret_cast<const u32x4a8*>(k + off);
    rg[p] = *reinterpret_cast<const u32x4a8*>(g + off);
  }
  const u32x4a8 kZero = {0u, 0u, 0u, 0u};

  // ---- per 32 channels: decay scan, scaled operands, Gram (channel
  // 32p + 8gq + i is Gram slot i of the lane) ----
  f32x4 Araw = zero4(), MrawT = zero4();
#pragma unroll
  for (int p = 0; p < NM / 2; ++p) {
    float qt[8], kt[8], kh[8], xq[8], xk[8], xg[8];
    unpack8(valid ? rq[p] : kZero, xq);
    unpack8(valid ? rk[p] : kZero, xk);
    unpack8(rg[p], xg);  // the decay of a padding token is zeroed below
    f16x8 kt16, kb16, qt16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = (valid ? gate_decay<GATE>(xg[i]) : 0.f) * kLog2e;
      const float G = row_inclusive_prefix_sum(x);
      const float E = __builtin_amdgcn_exp2f(G);
      const float Eh = __builtin_amdgcn_exp2f(-G);
      const float Eg = row_broadcast_last(E);  // e^gamma
      qt[i] = E * xq[i];
      kt[i] = E * xk[i];
      kh[i] = Eh * xk[i];
      kt16[i] = static_cast<Op>(kt[i]);
      kb16[i] = static_cast<Op>(kh[i] * Eg);  // e^(gamma - Gamma_r) k
      qt16[i] = static_cast<Op>(qt[i]);
      if (c16 == 15) s_eg[w][32 * p + 8 * gq + i] = E;  // e^gamma: the decay to the chunk's end
    }
    const int row = c16 * LDK + 32 * p + 8 * gq;  // one 16-byte store per lane and tile
    *reinterpret_cast<f16x8*>(&s_kt[w][row]) = kt16;
    *reinterpret_cast<f16x8*>(&s_kb[w][row]) = kb16;
    *reinterpret_cast<f16x8*>(&s_qt[w][row]) = qt16;
    bf16x8 kt_hi, kt_lo, kh_hi, kh_lo, qt_hi, qt_lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kt_hi[j] = static_cast<__bf16>(kt[j]);
      kt_lo[j] = static_cast<__bf16>(kt[j] - static_cast<float>(kt_hi[j]));
      kh_hi[j] = static_cast<__bf16>(kh[j]);
      kh_lo[j] = static_cast<__bf16>(kh[j] - static_cast<float>(kh_hi[j]));
      qt_hi[j] = static_cast<__bf16>(qt[j]);
      qt_lo[j] = static_cast<__bf16>(qt[j] - static_cast<float>(qt_hi[j]));
    }
    Araw = mma_16x16x32_bf16(kt_hi, kh_hi, Araw);
    Araw = mma_16x16x32_bf16(kt_hi, kh_lo, Araw);
    Araw = mma_16x16x32_bf16(kt_lo, kh_hi, Araw);
    MrawT = mma_16x16x32_bf16(kh_hi, qt_hi, MrawT);
    MrawT = mma_16x16x32_bf16(kh_lo, qt_hi, MrawT);
    MrawT = mma_16x16x32_bf16(kh_hi, qt_lo, MrawT);
  }
  if (gq == 0) s_beta[w][c16] = valid ? bf16_bits_to_f32(braw) : 0.f;
  __syncthreads();  // s_beta, s_kt, s_kb, s_qt, s_eg of both chunks visible
  if (w == 0) {
    // Qt of c1 in the record's fragment order (channel 16m + 4gq + i of the
    // lane's token), read back from LDS
#pragma unroll
    for (int p = 0; p < NM / 2; ++p) {
      f16x8 qv;
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[j] = s_qt[0][c16 * LDK + 16 * (2 * p + (j >> 2)) + 4 * gq + (j & 3)];
      *reinterpret_cast<f16x8*>(rec + L.q1 + static_cast<size_t>(p * 64 + l) * 16) = qv;
    }
  }

  // ---- mask: A strictly lower with row scale beta_r ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * gq + i, c = c16;
    s_A[w][r][c] = (c < r) ? s_beta[w][r] * Araw[i] : 0.f;
  }
  __syncthreads();

  // ---- Tm = (I + A)^-1, column c16 per lane, by forward substitution ----
  {
    float tc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == c16) ? 1.f : 0.f;
#pragma unroll
      for (int c = 0; c < r; ++c) acc -= s_A[w][r][c] * tc[c];
      tc[r] = acc;
    }
    if (gq == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_T[w][r][c16] = tc[r];
    }
  }
  __syncthreads();

  float tb[4], mf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * gq + i;
    tb[i] = s_T[w][c16][c] * s_beta[w][c];
    mf[i] = (c <= c16) ? MrawT[i] : 0.f;
  }

  // ---- W^T tiles: lane gets W[c16][16m + 4gq + i] ----
  float wv[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    f16x4 av, bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[i] = s_kt[w][(4 * gq + i) * LDK + 16 * m + c16];
      bv[i] = static_cast<_Float16>(tb[i]);
    }
    const f32x4 acc = mma_16x16x16_f16(av, bv, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[m][i] = acc[i];
  }

  const float* eg1 = s_eg[0];
  const float* eg2 = s_eg[1];
  if (w == 0) {
    // ---- c1: -W1, [Kb1 e^g2 | .], [M1 hi | lo], Tb1 ----
#pragma unroll
    for (int p = 0; p < NM / 2; ++p) {
      f16x8 x;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = static_cast<Op>(-wv[2 * p + (j >> 2)][j & 3]);
      *reinterpret_cast<f16x8*>(rec + L.w1 + static_cast<size_t>(p * 64 + l) * 16) = x;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const float e2 = eg2[16 * m + c16];
      f16x4 kv;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kv[i] = static_cast<Op>(static_cast<float>(s_kb[0][(4 * gq + i) * LDK + 16 * m + c16]) * e2);
      *reinterpret_cast<f16x4*>(rec + L.kb + static_cast<size_t>(m * 64 + l) * 16) = kv;
    }
    f16x8 mm;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mm[i] = static_cast<Op>(mf[i]);
      mm[i + 4] = static_cast<Op>(mf[i] - static_cast<float>(mm[i]));
    }
    *reinterpret_cast<f16x8*>(rec + L.m1 + static_cast<size_t>(l) * 16) = mm;
    *reinterpret_cast<bf16x8*>(rec + L.tb1 + static_cast<size_t>(l) * 16) = split_bf16(tb);
  } else {
    // ---- coupling tiles from Kb1 (wavefront 0's, in LDS): lane gets
    // C21[c16][4gq + i] and M21[c16][4gq + i] (products with Kb1 as the
    // first operand come out transposed) ----
    f32x4 C21T = zero4(), M21T = zero4();
#pragma unroll
    for (int p = 0; p < NM / 2; ++p) {
      f16x8 kb1, w2, q2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = 2 * p + (j >> 2), i = j & 3;
        const int ch = 16 * m + 4 * gq + i;
        kb1[j] = s_kb[0][c16 * LDK + ch];
        w2[j] = static_cast<Op>(wv[m][i]);
        q2[j] = s_qt[1][c16 * LDK + ch];
      }
      C21T = mma_16x16x32_f16(kb1, w2, C21T);
      M21T = mma_16x16x32_f16(kb1, q2, M21T);
    }
    // ---- c2: -W2 e^g1, Qt2 e^g1, [. | Kb2], [M21 | M2] hi and lo,
    // [Tb2 | -C21], e^(g1 + g2) ----
#pragma unroll
    for (int p = 0; p < NM / 2; ++p) {
      f16x8 x, y;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = 2 * p + (j >> 2), i = j & 3;
        const int ch = 16 * m + 4 * gq + i;
        const float e1 = eg1[ch];
        x[j] = static_cast<Op>(-wv[m][i] * e1);
        y[j] = static_cast<Op>(static_cast<float>(s_qt[1][c16 * LDK + ch]) * e1);
      }
      *reinterpret_cast<f16x8*>(rec + L.w2 + static_cast<size_t>(p * 64 + l) * 16) = x;
      *reinterpret_cast<f16x8*>(rec + L.q2 + static_cast<size_t>(p * 64 + l) * 16) = y;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      f16x4 kv;
#pragma unroll
      for (int i = 0; i < 4; ++i) kv[i] = s_kb[1][(4 * gq + i) * LDK + 16 * m + c16];
      *reinterpret_cast<f16x4*>(rec + L.kb + static_cast<size_t>(m * 64 + l) * 16 + 8) = kv;
    }
    f16x8 mh, ml;
    f16x4 cv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Op a = static_cast<Op>(M21T[i]), c = static_cast<Op>(mf[i]);
      mh[i] = a;
      ml[i] = static_cast<Op>(M21T[i] - static_cast<float>(a));
      mh[i + 4] = c;
      ml[i + 4] = static_cast<Op>(mf[i] - static_cast<float>(c));
      cv[i] = static_cast<Op>(-C21T[i]);
    }
    *reinterpret_cast<f16x8*>(rec + L.m2h + static_cast<size_t>(l) * 16) = mh;
    *reinterpret_cast<f16x8*>(rec + L.m2l + static_cast<size_t>(l) * 16) = ml;
    *reinterpret_cast<bf16x8*>(rec + L.tb2 + static_cast<size_t>(l) * 16) = split_bf16(tb);
    *reinterpret_cast<f16x4*>(rec + L.c21 + static_cast<size_t>(l) * 8) = cv;
    if (c16 == 15) {  // e^(gamma1 + gamma2), laid out as eg of kda_chunk_prep
      float* egp = reinterpret_cast<float*>(rec + L.eg) + gq * (DK / 4);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = eg1[16 * m + 4 * gq + i] * eg2[16 * m + 4 * gq + i];
        *reinterpret_cast<float4*>(egp + 4 * m) = make_float4(e[0], e[1], e[2], e[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sequential state pass.
// ---------------------------------------------------------------------------

template <int DK>
struct ChunkFrags {
  static constexpr int NM = DK / 16;
  f32x4 w[NM], q[NM], kb[NM];
  f32x4 mh, tb;
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
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint32_t off = static_cast<uint32_t>(m * 64 + l) * 16;
      w[m] = ld_at<f32x4>(rw, off);
      q[m] = ld_at<f32x4>(rq, off);
      kb[m] = ld_at<f32x4>(rk, off);
    }
    mh = ld_at<f32x4>(rm, static_cast<uint32_t>(l) * 16);
    tb = ld_at<f32x4>(rt, static_cast<uint32_t>(l) * 16);
#pragma unroll
    for (int m = 0; m < NM; ++m) eg[m] = ld_at<f32x4>(re, static_cast<uint32_t>(gq * NM + m) * 16);
  }

  // V rows 4gq + i of a chunk; `vchunk` (uniform) points at the chunk's first
  // token of this (b, h), vb[i] = ((4gq + i) * H * DV + col) * 4 (byte
  // offsets). Tokens at or past `valid` (a last partial chunk) read as zero.
  __device__ __forceinline__ void load_v(const float* vchunk, const uint32_t vb[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = ld_in_at(vchunk, vb[i]);
  }
  __device__ __forceinline__ void load_v_partial(const float* vchunk, const uint32_t vb[4], int gq,
                                                 int valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = (4 * gq + i < valid) ? ld_in_at(vchunk, vb[i]) : 0.f;
  }
};

// One chunk of the sequential pass on a dk x 16 state slice S (output layout):
// U = Tb V - W S,  O = Qt S + M U,  S <- Diag(e^gamma) S + Kb^T U.  Returns O.
template <int DK>
__device__ __forceinline__ f32x4 chunk_step(const ChunkFrags<DK>& cur, f32x4 (&S)[DK / 16]) {
  constexpr int NM = DK / 16;
  f32x4 U = zero4();
#pragma unroll
  for (int i = 0; i < 4; ++i) U = mma_16x16x4_f32(cur.tb[i], cur.vv[i], U);   // Ut = Tb V
  f32x4 O = zero4();
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      U = mma_16x16x4_f32(cur.w[m][i], S[m][i], U);                          // U = Ut - W S
      O = mma_16x16x4_f32(cur.q[m][i], S[m][i], O);                          // O = Qt S
    }
#pragma unroll
  for (int i = 0; i < 4; ++i) O = mma_16x16x4_f32(cur.mh[i], U[i], O);        // O += M U
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    S[m] = S[m] * cur.eg[m];
#pragma unroll
    for (int i = 0; i < 4; ++i) S[m] = mma_16x16x4_f32(cur.kb[m][i], U[i], S[m]);
  }
  return O;
}

// Sequential state pass for fp32 inputs: one wavefront per (b, h, 16-column
// slice of dv), reading the per-chunk records. MODE as for the bf16 pass.
template <typename OutT, int DK, int MODE>
__global__ __launch_bounds__(64) void kda_state_pass(const float* __restrict__ v,
                                                     const uint8_t* __restrict__ ws,
                                                     const float* S0, OutT* __restrict__ o,
                                                     float* ST, float* __restrict__ snap,
                                                     int64_t snap_chunks, int64_t T, int64_t H,
                                                     int64_t DV, int64_t NC, int64_t nslices,
                                                     int64_t nheads, RecordLayout L) {
  constexpr int NM = DK / 16;
  using Frags = ChunkFrags<DK>;
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
    for (int i = 0; i < 4; ++i) {
      if constexpr (MODE == kPassTransition)
        S[m][i] = (16 * m + 4 * gq + i == col) ? 1.f : 0.f;
      else
        S[m][i] = S0 ? S0[sbase + static_cast<size_t>(16 * m + 4 * gq + i) * DV] : 0.f;
    }
  constexpr bool kOut = MODE == kPassOutputs;

  // Uniform per-(b,h) bases; per-lane offsets fixed for the whole sequence.
  const uint8_t* rec0 = ws + static_cast<size_t>(head) * NC * L.bytes;
  const size_t hb = static_cast<size_t>(b * T * H + h) * DV;   // token 0 of (b, h)
  const float* vb = v + hb;
  OutT* ob = o + hb;
  const size_t chunk_elems = static_cast<size_t>(16 * H) * DV;
  // per-lane byte offsets of rows 4gq + i of a chunk (H * DV <= 2^25, so
  // 16 * H * DV elements of at most 4 bytes fit in 32 bits)
  uint32_t vbo[4], obo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t e = static_cast<uint32_t>((4 * gq + i) * H * DV + col);
    vbo[i] = e * static_cast<uint32_t>(sizeof(float));
    obo[i] = e * static_cast<uint32_t>(sizeof(OutT));
  }

  const int64_t NF = T / 16;  // full chunks
  // Full chunks: records prefetched one chunk ahead into two fragment
  // buffers whose roles alternate by unrolling (a register copy between
  // buffers would force a wait for the loads in flight); the last full chunk
  // is re-read past the end instead of branching around the load.
  auto fetch = [&](Frags& f, int64_t c) __attribute__((always_inline)) {
    c = c < NF - 1 ? c : NF - 1;
    f.load_record(rec0 + static_cast<size_t>(c) * L.bytes, L, l, gq);
    if constexpr (MODE == kPassTransition) {
      f.vv[0] = f.vv[1] = f.vv[2] = f.vv[3] = 0.f;
    } else {
      f.load_v(vb + static_cast<size_t>(c) * chunk_elems, vbo);
    }
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
    if constexpr (!kOut) return;
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
    Frags f0, f1;
    fetch(f0, 0);
    for (int64_t n = 0; n < NF; n += 2) {
      fetch(f1, n + 1);
      finish(n, chunk_step(f0, S));
      if (n + 1 >= NF) break;
      fetch(f0, n + 2);
      finish(n + 1, chunk_step(f1, S));
    }
  }
  if (NC > NF) {  // last partial chunk: padded tokens read as zero and are not stored
    const int valid = static_cast<int>(T - NF * 16);
    Frags f;
    f.load_record(rec0 + static_cast<size_t>(NF) * L.bytes, L, l, gq);
    if constexpr (MODE == kPassTransition) {
      f.vv[0] = f.vv[1] = f.vv[2] = f.vv[3] = 0.f;
    } else {
      f.load_v_partial(vb + static_cast<size_t>(NF) * chunk_elems, vbo, gq, valid);
    }
    const f32x4 O = chunk_step(f, S);
    if constexpr (kOut) {
      OutT* oc = ob + static_cast<size_t>(NF) * chunk_elems;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * gq + i < valid) st_out_at(oc, obo[i], O[i]);
    }
  }
  if (ST) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) ST[sbase + static_cast<size_t>(16 * m + 4 * gq + i) * DV] = S[m][i];
  }
}

// ---------------------------------------------------------------------------
// Sequential state pass, bf16 inputs: two loader wavefronts and a compute
// wavefront per (b, h, 16-column slice), advancing 32 tokens per step (or one
// compute wavefront for each of 2 or 4 slices of a head sharing the loaders,
// when the slices outnumber the compute units).
//
// The compute wavefront keeps its dk x 16 slice of S in registers and runs
// the sequential chain. Fed from global memory directly, a wavefront waits on
// its own prefetch loads (the compiler's wait placement in an unrolled
// prefetch loop leaves about one step of loads in flight, and HBM latency
// then sets the pace). Here the loader wavefronts stream each pair record and
// its V tiles from HBM into a ring of LDS slots, several steps ahead, with
// coalesced 16-byte loads (converting V to fp16, transposed for the MFMA
// operand); the compute wavefront only reads LDS. One LDS-only barrier per
// step keeps them in step. Barrier 0 follows the loader's prologue,
// barrier n + 1 ends step n:
//   prologue         the loader fills slots 0 .. kSlots-2 with pairs
//                    0 .. kSlots-2;
//   compute step n   reads pair n from its slot and processes it;
//   loader step n    between barriers n and n + 1, writes pair n + kSlots - 1
//                    into the slot of pair n - 1, which the compute wave read
//                    before barrier n; the write is complete at barrier n + 1,
//                    before its pair is read (after barrier n + kSlots - 1).
// Each loader keeps kStages pairs of its share of the loads in registers, so
// each pair's loads are issued kStages steps before they are written to LDS.
// Its loop runs a multiple of kStages steps with no exit in between (an exit
// inside made the compiler drain every load at the loop's back edge); the
// compute wave pads its barrier count to match.
//
// Per step the compute wavefront evaluates the pair lines of
// kda_chunk_prep_pair: 30 16x16x32 MFMAs (two of them bf16, for v's exact
// product), one decay multiply and one fp16 conversion of its state slice,
// two output stores and one barrier, against 36 MFMAs and two of each of the
// rest for two 16-token steps.
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// LDS-only release/acquire around a workgroup barrier: orders this wave's LDS
// accesses against the other wave's, without waiting for global loads. The
// scheduling barriers keep the instruction scheduler from moving work across
// steps (it would otherwise hoist the loader's use of loaded data to the top
// of the loop, where it must wait for every load in flight).
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

// Power-of-two scale of the bf16 path's state pass (see the compute wave):
// the slice's largest magnitude is kept in [kScaleLow, kScaleHigh], far
// inside the fp16 range ([2^-14, 65504] normal), with |e| <= kScaleMax.
constexpr float kScaleHigh = 16384.f;     // 2^14: fp16 holds 4x more
constexpr float kScaleLow = 0.0625f;      // 2^-4
constexpr int kScaleMax = 120;

// 2^x for an integer x in [-126, 127], exact.
__device__ __forceinline__ float pow2f(int x) { return __int_as_float((127 + x) << 23); }

// Largest value over the 64 lanes of the wavefront.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Largest magnitude in this lane's state slice, as a shallow tree of
// three-input maxima with absolute-value operands (NaN is ignored by the max).
template <int NM>
__device__ __forceinline__ float state_max(const f32x4 (&S)[NM]) {
  float part[NM];
#pragma unroll
  for (int k = 0; k < NM; ++k)
    part[k] = fmaxf(fmaxf(fmaxf(fabsf(S[k][0]), fabsf(S[k][1])), fabsf(S[k][2])), fabsf(S[k][3]));
#pragma unroll
  for (int w = 1; w < NM; w *= 2)
#pragma unroll
    for (int k = 0; k + w < NM; k += 2 * w) part[k] = fmaxf(part[k], part[k + w]);
  return part[0];
}

__device__ __forceinline__ float tile_max(float m, const f32x4& U) {
  return fmaxf(fmaxf(fmaxf(fmaxf(m, fabsf(U[0])), fabsf(U[1])), fabsf(U[2])), fabsf(U[3]));
}

template <int DK, int SPW>
struct Ring32Geom {
  static constexpr int kRec = DK == 128 ? 30720 : 18432;  // pair record bytes (pair_layout)
  static constexpr int kUnits = kRec / 1024;              // 16-byte record loads per lane
  // + two V^T tiles (16 columns x 16 tokens fp16) per slice of the workgroup,
  // rows padded to 10 dwords so that the loader's transposing writes hit 64
  // different LDS banks
  static constexpr int kVPitch = 40;                      // bytes per column row
  static constexpr int kVTile = 16 * kVPitch;             // bytes per chunk
  static constexpr int kSlot = kRec + SPW * 2 * kVTile;
  // Four slots let the loaders run up to three pairs ahead of the compute
  // wave, which absorbs the jitter of either side (measured on the 64K-token
  // workload: 3 slots 1.48-1.51 ms, 4 slots 1.46-1.48, 5 slots 1.50).
  static constexpr int kSlots = 4;
  // loader wavefronts: loader w loads record units j = w, w + kLoaders, ...;
  // the last one also loads V (two loads per slice; with four slices a V
  // wavefront of its own does, see Ring32Split). Each has its own load
  // counter, so each can keep more pairs in flight: kStages - 1 pairs of its
  // loads stay outstanding at each commit, within the 6-bit wait counter (one
  // loader 1.51 ms, two 1.48, three 1.52).
  static constexpr int kLoaders = 2;
  static constexpr int kUnitsPer = (kUnits + kLoaders - 1) / kLoaders;
  static constexpr int kStagesRaw = 1 + 63 / (kUnitsPer + 2 * SPW);  // + the V loads
  static constexpr int kStages = kStagesRaw > 5 ? 5 : kStagesRaw;
  static_assert((kStages - 1) * (kUnitsPer + 2 * SPW) <= 63, "loads in flight exceed the wait counter");
  // Outputs with SPW = 4: a token's 64 columns are adjacent in o, so the
  // compute wavefronts leave each step's output tiles in LDS as rows of the
  // pair's 32 tokens x 64 fp32, and store whole rows during the next step
  // (one request per line instead of one per slice and line). Two buffers,
  // by step parity. Measured: 1-7% off the pass with four slices; with two
  // (half-line rows for bf16 outputs) it cost up to 8%, so two slices keep
  // the direct stores.
  static constexpr bool kMergedOut = SPW == 4;
  static constexpr int kORow = SPW * 16 * 4;  // bytes per token row
  static constexpr int kOPair = 32 * kORow;   // bytes per pair
  static constexpr int kOStage = kMergedOut ? 2 * kOPair : 0;
};

// Outputs on a wavefront of their own (plain pass, output mode, one slice per
// workgroup, dk = 128). With one slice per compute unit the compute wavefront
// is the pass's critical path: it is busy about 92% of each step, the loaders
// 68-81% (shader-clock totals per wavefront, 64K-token workload). The output
// products (11 of the step's 30 MFMAs) and the output stores need the state
// only through its fp16 operand and [U1; U2], so the compute wavefront leaves
// those in LDS (two buffers by step parity) and an output wavefront forms and
// stores pair n's outputs during step n + 1, from the Q~ and M fragments it
// read from pair n's slot during step n.
//
// V on a wavefront of its own (four slices per workgroup, any mode that
// reads v). With four slices the V loader also loaded every slice's v and
// wrote its transposed tiles, and it set the pace: 128 heads of 128 x 128 over
// 8,192 tokens, busy 96% of each step while the other loader waited 81% of
// it. The V wavefront runs the loaders' loop (same stages, slots and
// barriers) with the V loads and tiles only, and the two record loaders split
// the record alone. Two slices keep V on a record loader: a fifth wavefront
// would halve the registers each may hold (the loaders' loads in flight need
// more than half of them).
template <int DK, int SPW, int MODE, bool SCALED>
struct Ring32Split {
  static constexpr bool kOn = DK == 128 && SPW == 1 && MODE == kPassOutputs && !SCALED;
  static constexpr int kXPair = (DK / 32 + 1) * 1024;  // fp16 state operand + [U1; U2] fragments
  static constexpr int kXStage = kOn ? 2 * kXPair : 0;
  static constexpr bool kVWave = SPW == 4 && MODE != kPassTransition;
  static constexpr int kVWaveIdx = Ring32Geom<DK, SPW>::kLoaders + SPW;  // after the compute waves
  static constexpr int kWaves = Ring32Geom<DK, SPW>::kLoaders + SPW + (kOn ? 1 : 0) + (kVWave ? 1 : 0);
};

// Time per 32-token step of a workgroup serving 2 or 4 slices, relative to one
// slice per workgroup (measured with 32 heads of 128 x 128 over 64K tokens,
// one workgroup per compute unit: 1.47, 1.65 and 2.04 ms).
constexpr double kSpw2StepCost = 1.12;
constexpr double kSpw4StepCost = 1.38;


// Whole-row V loads (two or four slices per workgroup). A token's columns
// of the group's slices are contiguous in v (64 or 128 bytes), so each load
// gives every lane 16 bytes (8 columns, piece j) of one token and covers
// whole rows: one request per token instead of one per slice. The lanes of
// tokens t and t ^ 1 are l and l ^ 8 (a DPP rotation by 8 within a 16-lane
// row); they swap half their pieces, and each writes four dwords (even token
// low, odd token high) of the transposed tiles: the even token's lane columns
// 0..3 of the piece, the odd token's lane columns 4..7.
template <int SPW>
struct VRows {
  static_assert(SPW == 2 || SPW == 4, "whole rows of two or four slices");
  static constexpr int kLoads = SPW;  // loads per pair and lane (32 tokens / (64 / (2 * SPW)))
  u32x4 x[kLoads];
  bool ok[kLoads];
  // piece (8 columns) and token (of the pair) of lane l in load i
  __device__ static int piece(int l) { return SPW == 4 ? (l & 7) : (l & 3); }
  __device__ static int token(int l, int i) {
    return SPW == 4 ? 8 * i + (l >> 3)
                    : 16 * i + (((l >> 3) & 1) | (((l >> 2) & 1) << 1) | ((l >> 4) << 2));
  }
};

template <int SPW>
struct VRowsSlot {};
template <>
struct VRowsSlot<2> {
  VRows<2> vr;
};

// Loads of pair c (tokens past T read the last token and are zeroed at
// commit); vp points at the pair's first token row, col at the lane's piece.
template <int SPW>
__device__ __forceinline__ void vrows_issue(VRows<SPW>& x, const uint16_t* vp, uint32_t vrow, uint32_t col,
                                            int64_t tmax, int64_t t0, int64_t T, int l) {
#pragma unroll
  for (int i = 0; i < VRows<SPW>::kLoads; ++i) {
    const int t = VRows<SPW>::token(l, i);
    const uint32_t tt = static_cast<uint32_t>(t < tmax ? t : tmax);
    x.x[i] = ld_at<u32x4>(vp, (tt * vrow + col) * 2u);
    x.ok[i] = t0 + t < T;
  }
}

// The transposed tiles of a pair: vt0 is the slot's first tile (slice 0,
// chunk 0); tile 2z + chunk holds column rows of kVPitch bytes.
template <int SPW, int kVPitch, int kVTile>
__device__ __forceinline__ void vrows_commit(const VRows<SPW>& x, uint8_t* vt0, bool von, int l) {
  const int j = VRows<SPW>::piece(l);
  const bool odd = ((l >> 3) & 1) != 0;
#pragma unroll
  for (int i = 0; i < VRows<SPW>::kLoads; ++i) {
    const int t = VRows<SPW>::token(l, i);  // chunk t >> 4, token pair (t & 15) >> 1
    const bool keep = x.ok[i] && von;
    // dword d of a piece holds columns 2d (low) and 2d + 1 (high); the even
    // token's lane needs the odd one's dwords 0, 1 and sends its dwords 2, 3
    // (scalars, not arrays: a select between array elements becomes an
    // indexed load from scratch)
    const uint32_t m0 = keep ? x.x[i][0] : 0u, m1 = keep ? x.x[i][1] : 0u;
    const uint32_t m2 = keep ? x.x[i][2] : 0u, m3 = keep ? x.x[i][3] : 0u;
    const uint32_t r0 = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(odd ? m0 : m2), 0x128, 0xf, 0xf, false));
    const uint32_t r1 = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(odd ? m1 : m3), 0x128, 0xf, 0xf, false));
    uint8_t* vt = vt0 + (2 * (j >> 1) + (t >> 4)) * kVTile + ((t & 15) >> 1) * 4;
    const int c0 = 8 * (j & 1) + (odd ? 4 : 0);  // first column of the four this lane writes
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t ew = odd ? (k < 2 ? r0 : r1) : (k < 2 ? m0 : m1);  // even token, this column pair
      const uint32_t ow = odd ? (k < 2 ? m2 : m3) : (k < 2 ? r0 : r1);  // odd token
      const uint32_t e = (k & 1) ? (ew >> 16) : (ew & 0xffffu);
      const uint32_t o2 = (k & 1) ? (ow & 0xffff0000u) : (ow << 16);
      *reinterpret_cast<uint32_t*>(vt + (c0 + k) * kVPitch) = e | o2;
    }
  }
}

template <int DK, int SPW>
struct Loader32Stage : VRowsSlot<SPW> {  // two slices: V in whole rows (vr)
  u32x4 r[Ring32Geom<DK, SPW>::kUnitsPer];
  u32x2 v0[SPW], v1[SPW];  // tokens 2a and 2a + 1, four columns of each slice (bf16)
  bool ok0, ok1;
};

template <int DK>
struct PairFrags {
  static constexpr int NM = DK / 16;
  f16x8 w1[NM / 2], w2[NM / 2], q1[NM / 2], q2[NM / 2];
  f16x8 kb[NM];
  f16x8 m1, m2h, m2l;
  bf16x8 tb1, tb2;
  f16x4 c21;
  bf16x4 v1, v2;
  f32x4 eg[NM];

  // vt: this slice's two V^T tiles (rows of kVPitch bytes, kVTile apart)
  template <int kVPitch, int kVTile>
  __device__ __forceinline__ void load(const uint8_t* slot, const uint8_t* vt, const PairLayout& L, int l,
                                       int gq, int c16) {
#pragma unroll
    for (int p = 0; p < NM / 2; ++p) {
      const uint32_t off = static_cast<uint32_t>(p * 64 + l) * 16;
      w1[p] = ld_at<f16x8>(slot + L.w1, off);
      w2[p] = ld_at<f16x8>(slot + L.w2, off);
      q1[p] = ld_at<f16x8>(slot + L.q1, off);
      q2[p] = ld_at<f16x8>(slot + L.q2, off);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      kb[m] = ld_at<f16x8>(slot + L.kb, static_cast<uint32_t>(m * 64 + l) * 16);
      eg[m] = ld_at<f32x4>(slot + L.eg, static_cast<uint32_t>(gq * NM + m) * 16);
    }
    const uint32_t lo = static_cast<uint32_t>(l) * 16;
    m1 = ld_at<f16x8>(slot + L.m1, lo);
    m2h = ld_at<f16x8>(slot + L.m2h, lo);
    m2l = ld_at<f16x8>(slot + L.m2l, lo);
    tb1 = ld_at<bf16x8>(slot + L.tb1, lo);
    tb2 = ld_at<bf16x8>(slot + L.tb2, lo);
    c21 = ld_at<f16x4>(slot + L.c21, static_cast<uint32_t>(l) * 8);
    const uint32_t vo = static_cast<uint32_t>(c16 * kVPitch + 8 * gq);
    v1 = ld_at<bf16x4>(vt, vo);
    v2 = ld_at<bf16x4>(vt + kVTile, vo);
  }
};

// With SPW > 1, one workgroup serves SPW consecutive 16-column slices of a
// head: one compute wavefront per slice, all reading the same record from the
// shared ring, and one wavefront loads every slice's V tiles (the second
// record loader, or with four slices a V wavefront of its own). A compute
// unit then advances SPW slices at once, for workloads with more slices than
// compute units. With one slice (dk = 128, plain output pass) an output
// wavefront forms and stores the outputs (Ring32Split).
//
// flags: one int per (b, h, slice), in the workspace after the records. The
// plain pass (SCALED = false) writes every slice's flag; the scaled pass
// (SCALED = true, SPW = 1) runs only the slices whose flag is set.
//
// MODE (kPassOutputs, kPassState or kPassTransition): the transition loads
// no V; the two state-only modes skip the output products and stores.
template <typename OutT, int DK, int SPW, bool SCALED, int MODE>
__global__ __launch_bounds__((64 * Ring32Split<DK, SPW, MODE, SCALED>::kWaves)) void kda_state_pass_ring32(
    const uint16_t* __restrict__ v, const uint8_t* __restrict__ ws, const float* S0,
    OutT* __restrict__ o, float* ST, float* __restrict__ snap, int64_t snap_pairs, int64_t T,
    int64_t H, int64_t DV, int64_t NPR, int64_t ngroups, int64_t nheads, PairLayout L,
    int* __restrict__ flags, float* __restrict__ E_out) {
  static_assert(!SCALED || SPW == 1, "the scaled pass serves one slice per workgroup");
  using G = Ring32Geom<DK, SPW>;
  using X = Ring32Split<DK, SPW, MODE, SCALED>;
  constexpr int NM = DK / 16;
  constexpr int kR = G::kSlots, kS = G::kStages;
  constexpr bool kMerged = MODE == kPassOutputs && G::kMergedOut;  // outputs staged as whole rows
  constexpr int kOStageBytes = kMerged ? G::kOStage : 0;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kR * G::kSlot + kOStageBytes + X::kXStage];
  uint8_t* const ostage = ring + kR * G::kSlot;
  uint8_t* const xbuf = ostage + kOStageBytes;  // compute -> output wavefront (X::kOn)

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, c16 = l & 15, gq = l >> 4;
  // XCD-aware numbering, as in kda_state_pass: all slice groups of a head
  // have ids congruent mod 8 and share one XCD's L2 for the head's records.
  const int64_t wgid = blockIdx.x;
  const int64_t xcd = wgid & 7, kk = wgid >> 3;
  const int64_t head = xcd + 8 * (kk / ngroups);
  const int64_t group = kk % ngroups;
  if (head >= nheads) return;  // whole workgroup
  if constexpr (SCALED) {
    if (flags[head * (DV / 16) + group] == 0) return;  // whole workgroup
  }
  const int64_t b = head / H, h = head % H;
  const uint8_t* rec0 = ws + static_cast<size_t>(head) * NPR * G::kRec;
  // kPassFE: the slices run over dk + dv columns, F's dk first, then E's dv;
  // v (and o) rows hold DVV = dv values
  const int64_t DVV = MODE == kPassFE ? DV - DK : DV;
  const size_t hb = static_cast<size_t>(b * T * H + h) * DVV;
  const size_t pair_elems = static_cast<size_t>(32 * H) * DVV;  // v or o elements per 32 tokens
  const int64_t NPF = T / 32;                                  // full pairs
  const int64_t NPS = (NPR + kS - 1) / kS * kS;                // loader steps (and barriers)

  constexpr int kLd = G::kLoaders;
  if constexpr (X::kVWave) {
    if (wave == X::kVWaveIdx) {
      // ---------------- V (four slices per workgroup) ----------------
      // The loaders' loop below (same stages, slots, steps and barriers)
      // with only a V part, in whole rows (VRows).
      static_assert(SPW == 4 && (DK / 16) % SPW == 0, "a group of four slices is all F or all E");
      const uint32_t vrow = static_cast<uint32_t>(H * DVV);  // elements per token
      // kPassFE: a group's slices are all F (v = 0: the loads read columns
      // 8j .. and are zeroed at commit) or all E, at column (s - dk / 16) * 16
      const int sl0 = static_cast<int>(group) * SPW;
      const bool von = MODE != kPassFE || sl0 >= DK / 16;
      const uint32_t col = static_cast<uint32_t>(
          (MODE == kPassFE ? (von ? (sl0 - DK / 16) * 16 : 0) : sl0 * 16) + 8 * VRows<SPW>::piece(l));
      const uint16_t* vb = v + hb;
      VRows<SPW> st[kS];
      auto issue = [&](VRows<SPW>& x, int64_t c) __attribute__((always_inline)) {
        const int64_t cc = c < NPR ? c : NPR - 1;
        vrows_issue<SPW>(x, vb + static_cast<size_t>(cc) * pair_elems, vrow, col, T - 1 - cc * 32, c * 32, T, l);
      };
      auto commit = [&](const VRows<SPW>& x, int64_t c) __attribute__((always_inline)) {
        vrows_commit<SPW, G::kVPitch, G::kVTile>(x, ring + static_cast<int>(c % kR) * G::kSlot + G::kRec, von, l);
      };
#pragma unroll
      for (int c = 0; c < kS; ++c) issue(st[c], c);
#pragma unroll
      for (int c = 0; c < kR - 1; ++c) {
        commit(st[c % kS], c);
        issue(st[c % kS], c + kS);
      }
      ring_barrier();
      for (int64_t n = 0; n < NPS; n += kS) {
#pragma unroll
        for (int k = 0; k < kS; ++k) {
          const int64_t c = n + k + kR - 1;
          commit(st[(k + kR - 1) % kS], c);
          issue(st[(k + kR - 1) % kS], c + kS);
          ring_barrier();
        }
      }
      return;
    }
  }
  if (wave < kLd) {
    // ---------------- loaders ----------------
    const bool has_v = !X::kVWave && wave == kLd - 1 && MODE != kPassTransition;
    // The slice groups of a head read the same record lines in the same
    // step. Each group starts its share of the units at a different place
    // (unit u of this loader's share is taken in turn (u + rot) mod
    // kUnitsPer), so that the groups' requests for a line do not arrive at
    // the L2 together (64K-token workload, 32 heads: 1.51 against 1.55 ms).
    static_assert(G::kUnits % kLd == 0, "every loader takes the same number of record units");
    const int rot = static_cast<int>((2 * group) % G::kUnitsPer);
    // V: lane -> tokens 2a, 2a + 1 of the pair (a = 0..15), columns 4cq ..
    // 4cq + 3 of each slice of the group
    const int va = l & 15, cq = l >> 4;
    const uint32_t vcol = static_cast<uint32_t>(group * SPW * 16 + 4 * cq);
    const uint32_t vrow = static_cast<uint32_t>(H * DVV);  // elements per token
    // kPassFE: slice s < dk / 16 is a column block of F (v = 0: its loads
    // read column 0 and are zeroed at commit), the others of E at column
    // (s - dk / 16) * 16
    auto vcol_of = [&](int z) __attribute__((always_inline)) -> uint32_t {
      if constexpr (MODE == kPassFE) {
        const int sl = static_cast<int>(group) * SPW + z;
        return static_cast<uint32_t>(sl >= DK / 16 ? (sl - DK / 16) * 16 + 4 * cq : 4 * cq);
      } else {
        return vcol + 16u * static_cast<uint32_t>(z);
      }
    };
    auto v_on = [&](int z) __attribute__((always_inline)) {
      return MODE != kPassFE || static_cast<int>(group) * SPW + z >= DK / 16;
    };
    const uint16_t* vb = v + hb;
    // two slices: whole rows (VRows); F or E for the whole group in kPassFE
    auto von2 = [&]() __attribute__((always_inline)) {
      return MODE != kPassFE || static_cast<int>(group) * SPW >= DK / 16;
    };
    auto col2 = [&]() __attribute__((always_inline)) {
      const int sl0 = static_cast<int>(group) * SPW;
      return static_cast<uint32_t>((MODE == kPassFE ? (von2() ? (sl0 - DK / 16) * 16 : 0) : sl0 * 16) +
                                   8 * VRows<2>::piece(l));
    };
    // Loads are unconditional (pairs past the end re-read the last one; V
    // tokens past T read the last token and are zeroed at commit): a branch
    // around them would make the compiler's wait counting conservative.
    auto issue = [&](Loader32Stage<DK, SPW>& st, int64_t c) __attribute__((always_inline)) {
      const int64_t cc = c < NPR ? c : NPR - 1;
      const uint8_t* src = rec0 + static_cast<size_t>(cc) * G::kRec;
#pragma unroll
      for (int u = 0; u < G::kUnitsPer; ++u) {
        const int j = wave + (u + rot) % G::kUnitsPer * kLd;
        st.r[u] = ld_at<u32x4>(src, static_cast<uint32_t>(j * 64 + l) * 16);
      }
      if constexpr (SPW == 2) {
        if (has_v)
          vrows_issue<2>(st.vr, vb + static_cast<size_t>(cc) * pair_elems, vrow, col2(), T - 1 - cc * 32,
                         c * 32, T, l);
      } else if (has_v) {
        const int64_t tmax = T - 1 - cc * 32;
        const uint32_t t0 = static_cast<uint32_t>(2 * va < tmax ? 2 * va : tmax);
        const uint32_t t1 = static_cast<uint32_t>(2 * va + 1 < tmax ? 2 * va + 1 : tmax);
        const uint16_t* vp = vb + static_cast<size_t>(cc) * pair_elems;
#pragma unroll
        for (int z = 0; z < SPW; ++z) {
          st.v0[z] = ld_at<u32x2>(vp, (t0 * vrow + vcol_of(z)) * 2u);
          st.v1[z] = ld_at<u32x2>(vp, (t1 * vrow + vcol_of(z)) * 2u);
        }
        st.ok0 = c * 32 + 2 * va < T;
        st.ok1 = c * 32 + 2 * va + 1 < T;
      }
    };
    // Commits are unconditional too: a pair past the end lands in a slot the
    // compute wave reads no more, and is never read.
    auto commit = [&](const Loader32Stage<DK, SPW>& st, int64_t c) __attribute__((always_inline)) {
      uint8_t* dst = ring + static_cast<int>(c % kR) * G::kSlot;
#pragma unroll
      for (int u = 0; u < G::kUnitsPer; ++u) {
        const int j = wave + (u + rot) % G::kUnitsPer * kLd;
        st_at<u32x4>(dst, static_cast<uint32_t>(j * 64 + l) * 16, st.r[u]);
      }
      if constexpr (SPW == 2) {
        if (has_v) vrows_commit<2, G::kVPitch, G::kVTile>(st.vr, dst + G::kRec, von2(), l);
      } else if (has_v) {
        // V^T[col][token], the exact bf16 values, one tile per chunk of the
        // pair (rows of G::kVPitch bytes), two tiles per slice: the compute
        // lane (c16, gq) reads tokens 4gq .. 4gq+3 of column c16. This lane
        // writes tokens 2a, 2a + 1 of its four columns of each slice, one
        // dword (two bf16) each.
#pragma unroll
        for (int z = 0; z < SPW; ++z) {
          uint8_t* vt = dst + G::kRec + (2 * z + (va >> 3)) * G::kVTile + (va & 7) * 4;
          const bool k0 = st.ok0 && v_on(z), k1 = st.ok1 && v_on(z);
          const uint32_t r0[2] = {k0 ? st.v0[z][0] : 0u, k0 ? st.v0[z][1] : 0u};
          const uint32_t r1[2] = {k1 ? st.v1[z][0] : 0u, k1 ? st.v1[z][1] : 0u};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t b0 = (c & 1) ? (r0[c >> 1] >> 16) : (r0[c >> 1] & 0xffffu);
            const uint32_t b1 = (c & 1) ? (r1[c >> 1] & 0xffff0000u) : (r1[c >> 1] << 16);
            *reinterpret_cast<uint32_t*>(vt + (4 * cq + c) * G::kVPitch) = b0 | b1;
          }
        }
      }
    };
    Loader32Stage<DK, SPW> st[kS];
#pragma unroll
    for (int c = 0; c < kS; ++c) issue(st[c], c);
#pragma unroll
    for (int c = 0; c < kR - 1; ++c) {
      commit(st[c % kS], c);
      issue(st[c % kS], c + kS);
    }
    ring_barrier();
    // step n writes pair n + kR - 1 and refills its stage kS pairs ahead; a
    // multiple of kS steps with no exit in between
    for (int64_t n = 0; n < NPS; n += kS) {
#pragma unroll
      for (int k = 0; k < kS; ++k) {
        const int64_t c = n + k + kR - 1;
        commit(st[(k + kR - 1) % kS], c);
        issue(st[(k + kR - 1) % kS], c + kS);
        ring_barrier();
      }
    }
    return;
  }

  if constexpr (X::kOn) {
    if (wave == kLd + SPW) {
      // ---------------- outputs (one slice per workgroup) ----------------
      // Step n reads the Q~ and M fragments of pair n from its slot (the
      // compute wavefront reads the same slot in the same step) and forms the
      // outputs of pair n - 1 from the fragments read in step n - 1 and the
      // compute wavefront's fp16 state operand and [U1; U2] of pair n - 1, in
      // the same product order as the compute wavefront's own output form.
      OutT* obo = o + hb;
      const uint32_t oto = static_cast<uint32_t>(c16 * H * DV + group * 16 + 4 * gq) *
                           static_cast<uint32_t>(sizeof(OutT));
      const size_t half = pair_elems / 2;
      PairFrags<DK> prev;
      ring_barrier();
      for (int64_t n = 0; n <= NPR; ++n) {
        PairFrags<DK> cur;
        if (n < NPR) {
          const uint8_t* slot = ring + static_cast<int>(n % kR) * G::kSlot;
          cur.template load<G::kVPitch, G::kVTile>(slot, slot + G::kRec, L, l, gq, c16);
        }
        if (n > 0) {
          const int64_t m = n - 1;
          const uint8_t* xb = xbuf + static_cast<int>(m & 1) * X::kXPair;
          f16x8 sh[NM / 2];
#pragma unroll
          for (int p = 0; p < NM / 2; ++p) sh[p] = ld_at<f16x8>(xb, static_cast<uint32_t>(p * 64 + l) * 16);
          const f16x8 u12 = ld_at<f16x8>(xb, static_cast<uint32_t>((NM / 2) * 64 + l) * 16);
          f16x8 u11;
#pragma unroll
          for (int i = 0; i < 4; ++i) u11[i] = u11[i + 4] = u12[i];
          f32x4 O1 = zero4(), O2 = zero4();
#pragma unroll
          for (int p = 0; p < NM / 2; ++p) {
            O1 = mma_16x16x32_f16(sh[p], prev.q1[p], O1);
            O2 = mma_16x16x32_f16(sh[p], prev.q2[p], O2);
          }
          O1 = mma_16x16x32_f16(u11, prev.m1, O1);
          O2 = mma_16x16x32_f16(u12, prev.m2h, O2);
          O2 = mma_16x16x32_f16(u12, prev.m2l, O2);
          OutT* oc = obo + static_cast<size_t>(m) * pair_elems;
          if (m < NPF) {
            st_out4_at(oc, oto, O1);
            st_out4_at(oc + half, oto, O2);
          } else {  // last, partial pair: tokens past T are not stored
            if (m * 32 + c16 < T) st_out4_at(oc, oto, O1);
            if (m * 32 + 16 + c16 < T) st_out4_at(oc + half, oto, O2);
          }
        }
        prev = cur;
        if (n < NPR) ring_barrier();
      }
      for (int64_t k = NPR; k < NPS; ++k) ring_barrier();  // match the loader's steps
      return;
    }
  }

  // ---------------- compute ----------------
  const int z = wave - kLd;  // this wavefront's slice within the group
  const int64_t slice = group * SPW + z;
  const int64_t col = slice * 16 + c16;
  const size_t sbase = static_cast<size_t>(head) * DK * DV + col;
  OutT* ob = o + hb;
  // outputs in transposed fragments: lane (c16, gq) holds token c16 of the
  // chunk, value columns slice*16 + 4gq .. +3
  const uint32_t obt =
      static_cast<uint32_t>(c16 * H * DV + slice * 16 + 4 * gq) * static_cast<uint32_t>(sizeof(OutT));
  const size_t chunk_elems = pair_elems / 2;
  float* snap_b = nullptr;
  if (snap_pairs > 0) {
    const int64_t ns = NPF / snap_pairs;
    snap_b = snap + (static_cast<size_t>(b * ns) * H + h) * DK * DV + slice * 16;
  }
  // the slice in [dk, DV] row-major fp32 at a uniform base: per-lane byte
  // offsets of rows 4gq + i of channel group 0 (DK * DV * 4 < 2^32)
  // kPassFE: F's slices (slice < dk / 16) are dk wide, E's dv wide
  const bool fe_f = MODE == kPassFE && slice < DK / 16;
  const uint32_t srow = static_cast<uint32_t>(MODE == kPassFE ? (fe_f ? DK : DVV) : DV) * 4u;
  const uint32_t slane = static_cast<uint32_t>(4 * gq) * srow + static_cast<uint32_t>(c16) * 4u;

  // The state and update products take fp16 operands, so the state S and
  // the update U must stay inside the fp16 range; v enters exact (bf16)
  // through Tb V in fp32. The plain pass (SCALED = false) runs as is. A
  // value past the fp16 range becomes an infinity there, and from then on
  // the state holds a non-finite entry for good (the decay and the products
  // keep infinities and NaN); values far below the range (all of |S| <
  // kScaleLow at the end) lose fp16 precision. Either way the final state
  // shows it: the plain pass then leaves S_T unwritten (so an in-place S0
  // survives) and raises the slice's flag, and the scaled pass
  // (SCALED = true, launched after it) redoes exactly the flagged slices
  // from S0. Ordinary inputs pay one check per slice; NaN or infinite
  // inputs run twice, with the same result.
  //
  // Scaled pass: the slice is held as S * 2^-e (fp32) with a wave-uniform
  // integer e, and every step checks the largest |S 2^-e| and |U 2^-e|
  // before the update products use them. Above kScaleHigh, or below
  // kScaleLow in every lane, e moves so that the slice's largest magnitude
  // lands in [2^5, 2^6) and the step's state products are redone. Powers of
  // two scale exactly; while e = 0 the arithmetic is that of the plain pass.
  f32x4 S[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (MODE == kPassTransition)
        S[m][i] = (16 * m + 4 * gq + i == col) ? 1.f : 0.f;
      else if constexpr (MODE == kPassFE)  // F from the identity, E from zero
        S[m][i] = (fe_f && 16 * m + 4 * gq + i == col) ? 1.f : 0.f;
      else
        S[m][i] = S0 ? S0[sbase + static_cast<size_t>(16 * m + 4 * gq + i) * DV] : 0.f;
    }
  constexpr bool kOut = MODE == kPassOutputs;
  constexpr bool kOutHere = kOut && !X::kOn;  // this wavefront forms and stores the outputs
  int e = 0;
  float dn = 1.f, up = 1.f;  // 2^-e, 2^e
  int64_t next_snap = snap_pairs;
  auto store_slice = [&](float* base) __attribute__((always_inline)) {
    // an opaque copy keeps the 32 address computations inside this rare path
    // (hoisted out of the loop they stay live for the whole sequence)
    uint32_t lane_off = slane;
    asm volatile("" : "+v"(lane_off));
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) st_at<float>(base, lane_off + (16 * m + i) * srow, S[m][i] * up);
  };
  // Stores the staged outputs of pair m: compute wavefront z takes tokens
  // z * 32/SPW .. of the pair, whole rows of 16-byte pieces (64 / pieces
  // per row tokens per instruction); tokens past T are not stored.
  auto store_staged = [&](int64_t m) __attribute__((always_inline)) {
    if constexpr (kMerged) {
      constexpr int kPieces = G::kORow / 16;         // 16-byte pieces per row
      constexpr int kTokInstr = 64 / kPieces;        // tokens per instruction
      constexpr int kTokWave = 32 / SPW;             // tokens per wavefront
      const uint8_t* src = ostage + static_cast<int>(m & 1) * G::kOPair;
      OutT* om = ob + static_cast<size_t>(m) * pair_elems;
      const int piece = l % kPieces;
#pragma unroll
      for (int i = 0; i < kTokWave / kTokInstr; ++i) {
        const int tok = z * kTokWave + i * kTokInstr + l / kPieces;
        const f32x4 x = ld_at<f32x4>(src, static_cast<uint32_t>(tok * G::kORow + piece * 16));
        const uint32_t off = static_cast<uint32_t>(tok * H * DV + group * SPW * 16 + 4 * piece) *
                             static_cast<uint32_t>(sizeof(OutT));
        if (m < NPF || m * 32 + tok < T) st_out4_at(om, off, x);
      }
    }
  };
  ring_barrier();
  for (int64_t n = 0; n < NPR; ++n) {
    if (n > 0) store_staged(n - 1);  // staged last step, visible since the barrier
    PairFrags<DK> f;
    const uint8_t* slot = ring + static_cast<int>(n % kR) * G::kSlot;
    f.template load<G::kVPitch, G::kVTile>(slot, slot + G::kRec + 2 * z * G::kVTile, L, l, gq, c16);
    // Tb V of both chunks: v exact in bf16 (repeated in both halves of the
    // contraction) against Tb's high and low bf16 parts
    bf16x8 vv1, vv2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vv1[i] = vv1[i + 4] = f.v1[i];
      vv2[i] = vv2[i + 4] = f.v2[i];
    }
    f32x4 TV1 = zero4(), TV2 = zero4();  // v = 0 for the transition
    if constexpr (MODE != kPassTransition) {
      TV1 = mma_16x16x32_bf16(f.tb1, vv1, zero4());
      TV2 = mma_16x16x32_bf16(f.tb2, vv2, zero4());
    }
    f16x8 cz;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cz[i] = f.c21[i];
      cz[i + 4] = static_cast<_Float16>(0.f);
    }
    f16x8 sh[NM / 2];
    f32x4 U1, U2, O1, O2;
    float mx = 0.f;
    // the products that read the state: U1, U2 and the state parts of O1, O2
    auto state_products = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < NM / 2; ++p)
#pragma unroll
        for (int j = 0; j < 8; ++j) sh[p][j] = static_cast<_Float16>(S[2 * p + (j >> 2)][j & 3]);
      float ms = 0.f;
      if constexpr (SCALED) ms = state_max(S);  // independent of the products below
      U1 = TV1 * dn;                                              // Tb1 V1
      U2 = TV2 * dn;                                              // Tb2 V2
      O1 = zero4();
      O2 = zero4();
#pragma unroll
      for (int p = 0; p < NM / 2; ++p) {
        U1 = mma_16x16x32_f16(f.w1[p], sh[p], U1);                // - W1 S0
        U2 = mma_16x16x32_f16(f.w2[p], sh[p], U2);                // - W2 e^g1 S0
        if constexpr (kOutHere) {
          O1 = mma_16x16x32_f16(sh[p], f.q1[p], O1);              // (Qt1 S0)^T
          O2 = mma_16x16x32_f16(sh[p], f.q2[p], O2);              // (Qt2 e^g1 S0)^T
        }
      }
      f16x8 uz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uz[i] = static_cast<_Float16>(U1[i]);
        uz[i + 4] = static_cast<_Float16>(0.f);
      }
      U2 = mma_16x16x32_f16(cz, uz, U2);                          // - C21 U1
      if constexpr (SCALED) mx = tile_max(tile_max(ms, U1), U2);
    };
    // NaN never counts (the max ignores it) and an infinite value does not
    // either: both propagate unscaled
    auto out_of_range = [&]() __attribute__((always_inline)) {
      const float fin = mx <= 3.4028235e38f ? mx : 0.f;
      return __any(fin > kScaleHigh) || (!__any(mx >= kScaleLow) && __any(fin > 0.f));
    };
    state_products();
    if constexpr (SCALED) {
      if (out_of_range()) {
        // shift so that the slice's largest finite magnitude is in
        // [2^5, 2^6), then redo the products (a branch, not a loop around
        // the common path: a loop there makes the compiler wait for every
        // fragment read before the first product)
        for (int redo = 0; redo < 3; ++redo) {
          const float fin = mx <= 3.4028235e38f ? mx : 0.f;
          const int x = __builtin_amdgcn_frexp_expf(wave_max(fin));
          int en = e - (6 - x);
          en = en < -kScaleMax ? -kScaleMax : (en > kScaleMax ? kScaleMax : en);
          const int d = __builtin_amdgcn_readfirstlane(e - en);
          if (d == 0) break;  // held at the limit
          e -= d;
          dn = pow2f(-e);
          up = pow2f(e);
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[m][i] = __builtin_amdgcn_ldexpf(S[m][i], d);
          state_products();
          if (!out_of_range()) break;
        }
      }
    }
    f16x8 u11, u12;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 x = static_cast<_Float16>(U1[i]);
      u11[i] = x;
      u11[i + 4] = x;
      u12[i] = x;
      u12[i + 4] = static_cast<_Float16>(U2[i]);
    }
    if constexpr (X::kOn) {  // the output wavefront's operands, read during the next step
      uint8_t* xb = xbuf + static_cast<int>(n & 1) * X::kXPair;
#pragma unroll
      for (int p = 0; p < NM / 2; ++p) st_at<f16x8>(xb, static_cast<uint32_t>(p * 64 + l) * 16, sh[p]);
      st_at<f16x8>(xb, static_cast<uint32_t>((NM / 2) * 64 + l) * 16, u12);
    }
    if constexpr (kOutHere) {
      O1 = mma_16x16x32_f16(u11, f.m1, O1);                       // + (M1 U1)^T
      O2 = mma_16x16x32_f16(u12, f.m2h, O2);                      // + ([M21 | M2] [U1; U2])^T
      O2 = mma_16x16x32_f16(u12, f.m2l, O2);
    }
    // S = Diag(e^(g1+g2)) S + [Kb1 e^g2 | Kb2]^T [U1; U2] (accumulator input
    // is the VALU product)
#pragma unroll
    for (int m = 0; m < NM; ++m) S[m] = mma_16x16x32_f16(f.kb[m], u12, S[m] * f.eg[m]);
    if constexpr (kOutHere) {
      if constexpr (SCALED) {
        O1 *= up;
        O2 *= up;
      }
      if constexpr (kMerged) {
        // this slice's columns of tokens c16 and 16 + c16; stored next step
        uint8_t* dst = ostage + static_cast<int>(n & 1) * G::kOPair;
        const uint32_t col = static_cast<uint32_t>(z * 64 + gq * 16);
        st_at<f32x4>(dst, static_cast<uint32_t>(c16 * G::kORow) + col, O1);
        st_at<f32x4>(dst, static_cast<uint32_t>((16 + c16) * G::kORow) + col, O2);
      } else {
        OutT* oc = ob + static_cast<size_t>(n) * pair_elems;
        if (n < NPF) {
          st_out4_at(oc, obt, O1);
          st_out4_at(oc + chunk_elems, obt, O2);
        } else {  // last, partial pair: tokens past T are not stored
          if (n * 32 + c16 < T) st_out4_at(oc, obt, O1);
          if (n * 32 + 16 + c16 < T) st_out4_at(oc + chunk_elems, obt, O2);
        }
      }
    }
    if (kOut && n + 1 == next_snap && n < NPF) {
      store_slice(snap_b + static_cast<size_t>(n / snap_pairs) * H * DK * DV);
      next_snap += snap_pairs;
    }
    ring_barrier();
  }
  store_staged(NPR - 1);  // the last pair, staged before the last barrier
  for (int64_t k = NPR; k < NPS; ++k) ring_barrier();  // match the loader's steps
  if constexpr (!SCALED) {
    // suspect: a non-finite entry anywhere in the slice (the sum keeps it),
    // or every entry below kScaleLow while some are still normal fp32 values.
    // Once fp16 operands underflow, the plain pass keeps only the decay of the
    // fp32 state (an upper bound on its size, since the rest of each step is
    // a contraction for keys of norm at most 1), so a state that ends below
    // the smallest normal fp32 value is below fp32's range however it is
    // computed (e.g. the transition of a long span), and is not redone.
    float sum = 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += fabsf(S[m][i]);
    const float ms = state_max(S);
    const bool suspect = __any(!(sum <= 3.4028235e38f)) ||
                         (!__any(ms >= kScaleLow) && __any(ms >= 1.17549435e-38f));
    if (l == 0) flags[head * (DV / 16) + slice] = suspect ? 1 : 0;
    if (suspect) return;
  }
  if constexpr (MODE == kPassFE) {
    if (fe_f)
      store_slice(ST + static_cast<size_t>(head) * DK * DK + slice * 16);
    else
      store_slice(E_out + static_cast<size_t>(head) * DK * DVV + (slice - DK / 16) * 16);
  } else {
    if (ST) store_slice(ST + static_cast<size_t>(head) * DK * DV + slice * 16);
  }
}

// T = 0: the final state is the initial one (or zeros).
__global__ void kda_copy_state(const float* S0, float* ST, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) ST[i] = S0 ? S0[i] : 0.f;
}

// The transition of an empty span: n / (d * d) identity matrices of d x d.
__global__ void kda_identity_states(float* F, int64_t d, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) F[i] = (i % d) == ((i / d) % d) ? 1.f : 0.f;
}

template <typename InT, int DK, int GATE>
hipError_t launch_prep_typed(const ChunkFwdArgs& a, hipStream_t stream) {
  if constexpr (!kIsF32<InT>) {  // bf16 inputs: one record per pair of chunks
    const PairLayout L = pair_layout(DK);
    if (L.bytes != Ring32Geom<DK, 1>::kRec) return hipErrorInvalidValue;
    const int64_t NPR = (a.T + 31) / 32;
    const int64_t blocks = a.B * NPR * a.H;
    hipLaunchKernelGGL((kda_chunk_prep_pair<DK, GATE>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(128), 0, stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.g),
                       static_cast<const uint16_t*>(a.beta), static_cast<uint8_t*>(a.workspace),
                       a.T, a.H, NPR, L);
    return hipGetLastError();
  } else {
    const RecordLayout L = record_layout(DK);
    const int64_t NC = (a.T + 15) / 16;
    const int64_t blocks = a.B * NC * a.H;
    hipLaunchKernelGGL((kda_chunk_prep<DK, GATE>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(64), 0, stream, static_cast<const float*>(a.q),
                       static_cast<const float*>(a.k), static_cast<const float*>(a.g),
                       static_cast<const float*>(a.beta), static_cast<uint8_t*>(a.workspace), a.T,
                       a.H, NC, L);
    return hipGetLastError();
  }
}

// Snapshots are taken only when at least one falls inside the sequence.
inline bool wants_snapshots(const ChunkFwdArgs& a) {
  return a.snapshots != nullptr && a.snapshot_every > 0 && a.T >= a.snapshot_every;
}

template <typename OutT, int DK, int SPW, bool SCALED, int MODE>
hipError_t launch_ring32(const ChunkFwdArgs& a, int64_t snap_pairs, hipStream_t stream) {
  using G = Ring32Geom<DK, SPW>;
  const PairLayout P = pair_layout(DK);
  if (P.bytes != G::kRec) return hipErrorInvalidValue;  // layout and ring disagree
  const int64_t NPR = (a.T + 31) / 32;
  const int64_t ngroups = a.dv / 16 / SPW;
  const int64_t nheads = a.B * a.H;
  const int64_t blocks = 8 * ngroups * ((nheads + 7) / 8);
  int* flags = reinterpret_cast<int*>(static_cast<uint8_t*>(a.workspace) +
                                      static_cast<size_t>(nheads * NPR) * G::kRec);
  hipLaunchKernelGGL((kda_state_pass_ring32<OutT, DK, SPW, SCALED, MODE>),
                     dim3(static_cast<uint32_t>(blocks)),
                     dim3(64 * Ring32Split<DK, SPW, MODE, SCALED>::kWaves), 0, stream,
                     static_cast<const uint16_t*>(a.v), static_cast<const uint8_t*>(a.workspace),
                     a.S0, static_cast<OutT*>(a.o), a.S_T, snap_pairs > 0 ? a.snapshots : nullptr,
                     snap_pairs, a.T, a.H, a.dv, NPR, ngroups, nheads, P, flags, a.E_out);
  return hipGetLastError();
}

// The plain pass with SPW slices per workgroup, then the scaled pass over the
// slices it flagged (one per workgroup; the others exit at once).
template <typename OutT, int DK, int SPW, int MODE>
hipError_t launch_ring32_pair(const ChunkFwdArgs& a, int64_t snap_pairs, hipStream_t stream) {
  const hipError_t e = launch_ring32<OutT, DK, SPW, false, MODE>(a, snap_pairs, stream);
  if (e != hipSuccess) return e;
  return launch_ring32<OutT, DK, 1, true, MODE>(a, snap_pairs, stream);
}

// Slices per state-pass workgroup (1, 2 or 4, a divisor of the slice count).
// Each workgroup runs the sequential chains of its slices. Estimated time:
// (workgroups per compute unit, rounded up) x (relative time per step).
// Workgroups that share a compute unit (dk = 64 rings leave room for two)
// share its issue slots and LDS as well, so the estimate counts them as
// taking turns. This picks the fastest variant in every case measured: 32 to
// 256 heads, dk 64 and 128, dv 64 and 128 (e.g. 64 heads of 128 x 128: 0.205,
// 0.136, 0.159 ms for 1, 2, 4 slices; 128 heads: 0.770, 0.482, 0.377 ms).
inline int choose_slices_per_wg(int64_t nheads, int64_t nslices, int cus) {
  const double step[3] = {1.0, kSpw2StepCost, kSpw4StepCost};
  int best = 1;
  double best_t = 0;
  for (int i = 0; i < 3; ++i) {
    const int spw = 1 << i;
    if (nslices % spw) continue;
    const int64_t wgs = nheads * (nslices / spw);
    const double t = static_cast<double>((wgs + cus - 1) / cus) * step[i];
    if (i == 0 || t < best_t) {
      best = spw;
      best_t = t;
    }
  }
  return best;
}

// `a.dv` is the column count of the pass: the value dimension, or dk for
// the transition.
template <typename InT, typename OutT, int DK, int MODE>
hipError_t launch_pass_typed(const ChunkFwdArgs& a, hipStream_t stream) {
  const int64_t nslices = a.dv / 16;
  const int64_t nheads = a.B * a.H;
  const int64_t blocks = 8 * nslices * ((nheads + 7) / 8);
  const int64_t snap_chunks =
      MODE == kPassOutputs && wants_snapshots(a) ? a.snapshot_every / 16 : 0;
  if constexpr (!kIsF32<InT>) {  // bf16 inputs: 32 tokens per step
    const int64_t snap_pairs = snap_chunks / 2;
    if constexpr (MODE != kPassOutputs && MODE != kPassFE) {
      return launch_ring32_pair<OutT, DK, 1, MODE>(a, 0, stream);
    } else {
      int dev = 0, cus = 256;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
      switch (choose_slices_per_wg(nheads, nslices, cus > 0 ? cus : 1)) {
        case 4: return launch_ring32_pair<OutT, DK, 4, MODE>(a, snap_pairs, stream);
        case 2: return launch_ring32_pair<OutT, DK, 2, MODE>(a, snap_pairs, stream);
        default: return launch_ring32_pair<OutT, DK, 1, MODE>(a, snap_pairs, stream);
      }
    }
  } else {
    const RecordLayout L = record_layout(DK);
    const int64_t NC = (a.T + 15) / 16;
    hipLaunchKernelGGL((kda_state_pass<OutT, DK, MODE>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(64), 0, stream, static_cast<const float*>(a.v),
                       static_cast<const uint8_t*>(a.workspace), a.S0, static_cast<OutT*>(a.o),
                       a.S_T, snap_chunks > 0 ? a.snapshots : nullptr, snap_chunks, a.T, a.H, a.dv,
                       NC, nslices, nheads, L);
    return hipGetLastError();
  }
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

template <typename InT, typename OutT, int MODE = kPassOutputs>
hipError_t launch_pass_dk(const ChunkFwdArgs& a, hipStream_t s) {
  return a.dk == 64 ? launch_pass_typed<InT, OutT, 64, MODE>(a, s)
                    : launch_pass_typed<InT, OutT, 128, MODE>(a, s);
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

hipError_t launch_chunk_transition(const ChunkFwdArgs& a, float* F, float* E, hipStream_t stream) {
  if (a.B * a.H == 0) return hipSuccess;
  const bool in32 = a.in_dtype == 0;
  if (a.T == 0) {  // F = I, E = 0
    const int64_t n = a.B * a.H * a.dk;
    if (F)
      hipLaunchKernelGGL(kda_identity_states, dim3(static_cast<uint32_t>((n * a.dk + 255) / 256)),
                         dim3(256), 0, stream, F, a.dk, n * a.dk);
    if (E)
      hipLaunchKernelGGL(kda_copy_state, dim3(static_cast<uint32_t>((n * a.dv + 255) / 256)),
                         dim3(256), 0, stream, nullptr, E, n * a.dv);
    return hipGetLastError();
  }
  ChunkFwdArgs t = a;
  t.S0 = nullptr;
  t.o = nullptr;
  t.snapshots = nullptr;
  t.snapshot_every = 0;
  if (F && E && !in32) {
    // both in one pass over dk + dv columns: [F | E] is one state, from
    // [I | 0] with v taken as [0 | v] (each column evolves on its own), so
    // the slices of F and E share the record stream of their head
    t.dv = a.dk + a.dv;
    t.S_T = F;
    t.E_out = E;
    return launch_pass_dk<uint16_t, float, kPassFE>(t, stream);
  }
  if (F) {  // dk columns from the identity, v = 0
    t.dv = a.dk;
    t.S_T = F;
    const hipError_t e = in32 ? launch_pass_dk<float, float, kPassTransition>(t, stream)
                              : launch_pass_dk<uint16_t, float, kPassTransition>(t, stream);
    if (e != hipSuccess) return e;
  }
  if (E) {  // the state reached from zero
    t.dv = a.dv;
    t.S_T = E;
    return in32 ? launch_pass_dk<float, float, kPassState>(t, stream)
                : launch_pass_dk<uint16_t, float, kPassState>(t, stream);
  }
  return hipSuccess;
}

hipError_t launch_chunk_fwd(const ChunkFwdArgs& a, hipStream_t stream) {
  const hipError_t e = launch_chunk_prep(a, stream);
  if (e != hipSuccess) return e;
  return launch_chunk_state_pass(a, stream);
}

// ---------------------------------------------------------------------------
// Built-in scratch of the no-allocation forward: room for the prep records
// and the state pass's flags of one call. Each device holds its own copy. The
// array's name is a host-side stand-in in host code, so kernels receive the
// device address from hipGetSymbolAddress, taken once per device with that
// device current. Every call on a device uses the same array: calls that
// overlap in time on one device race. Nothing in it needs clearing: the prep
// writes every record before the pass reads it, and the plain pass writes
// every flag before the scaled pass reads it.
// ---------------------------------------------------------------------------
namespace {

__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kda
