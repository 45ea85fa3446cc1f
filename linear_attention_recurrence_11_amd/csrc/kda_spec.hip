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
// Verify (kda_spec_verify_cols) gives each wavefront 16 value columns of one
// (request, head) unit with all dk rows: every column of the state evolves on
// its own, so the sums over rows are cross-lane exchanges and a token needs
// no barrier. Commit (kda_spec_kernel) runs up to 1024 persistent 1024-thread
// workgroups that take the units in turn and load the next unit's state
// while replaying the current one (spec_threads, kCommitGrid); thread t owns
// float4 column group cg = t % (dv/4) of rows rg + RG*j, as in the decode
// step, with two barriers per token (partial reductions written, u
// published). Both keep their part of S in registers across all tokens and
// stage a block of tokens' inputs in LDS at once (commit loads a unit's
// first block one unit ahead, beside that unit's state), so no token waits
// on a global load of its own. Verify falls back to kda_spec_kernel (one
// 256-thread workgroup per unit) when its inputs are not 16-byte aligned.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// Threads per workgroup of kda_spec_kernel (commit, and verify for inputs
// that are not 16-byte aligned). Verify reads the state once and synchronises
// every token, which favours small workgroups; commit also writes the state back,
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

// ---- verify by column slices ---------------------------------------------
// Every value column of the state evolves on its own: the decay scales rows,
// and the erase and the write of column c read only column c, v_c and the
// token's k, q and beta (the decode step's per-column form). So a wavefront
// that holds all dk rows of 16 columns needs no other wavefront: its sums
// over rows are cross-lane exchanges, with no LDS and no barrier per token.
//
// A workgroup is 4 such wavefronts, 64 columns of one (request, head) unit
// (all of them for dv = 64). The token inputs of a block of TB tokens are
// staged in LDS at once (q, k, e^gate and the workgroup's v columns, widened
// to fp32), behind one barrier; the next block's inputs are loaded into
// registers before the current block's tokens run. The loads that a staging
// waits for are older than the previous block's output stores, but the wait
// also covers those stores (the memory counter drains in issue order and
// their number is not fixed), so blocks are as long as the drafts allow:
// TB = 8 up to 8 drafts, 16 beyond (measured: 16 costs 3% at one draft, and
// saves 9% at twelve).
//
// Lane l = 16 rho + 4 i + cq (rho the 16-lane row, i and cq in 0..3) holds
// columns 4 cq .. + 3 of its wavefront's 16 in rows R rg .. + R - 1, where
// rg = 4 rho + i and R = dk / 16. The row sums of a token are reduced and
// scattered at once: after the exchanges, the lanes of row rho hold the sums
// of column 4 cq + rho, where that column's u and output are formed; u then
// returns to all four rows for the update.
//
// Measured at 256 requests x 32 heads, d = 128, bf16 inputs: 115, 142, 175
// and 227 us for 1, 4, 8 and 12 drafts, against 129, 171, 216 and 262 us for
// kda_spec_kernel. Workgroups of 8 wavefronts (a whole unit) gave 117, 149,
// 183 and 271 us; a persistent grid loading the next unit's state ahead
// needs about 150 registers (one workgroup per compute unit) and took 128 us
// for one draft but 181 us for four.

constexpr int kVerifyCols = 64;  // value columns per workgroup (4 wavefronts)

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t x) { return __builtin_bit_cast(float, x); }
// A copy in a register of its own (identity quad permutation): the lane
// swaps below exchange two registers, and one value passed as both operands
// would be one register.
__device__ __forceinline__ float own_copy(float x) { return dpp_move<0xE4>(x); }

// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second. For a and b it returns, summed: in rows 0 and
// 2, a over rows {0, 1} and {2, 3}; in rows 1 and 3, b over the same pairs.
__device__ __forceinline__ float swap_add16(float a, float b) {
  const auto p = __builtin_amdgcn_permlane16_swap(fbits(a), fbits(b), false, false);
  return bitsf(p[0]) + bitsf(p[1]);
}
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with
// the lower 32 of its second: summed, the low half holds a over both halves
// and the high half b over both halves.
__device__ __forceinline__ float swap_add32(float a, float b) {
  const auto p = __builtin_amdgcn_permlane32_swap(fbits(a), fbits(b), false, false);
  return bitsf(p[0]) + bitsf(p[1]);
}
// Sum over the four lanes 4 i + cq, i = 0..3, of each row (rotations by 8,
// then 4: each step adds a pair of values that both of its lanes hold, so
// the four lanes end with the same bits).
__device__ __forceinline__ float sum_quads_of_row(float x) {
  x += dpp_move<0x128>(x);  // row_ror:8
  x += dpp_move<0x124>(x);  // row_ror:4
  return x;
}

// FUSED: the same kernel first replays the accepted prefix of the previous
// round's logged tokens (k1, v1, g1, beta1; accepted[n] of T1, as in the
// commit), writes the advanced state back once, and then verifies the drafts
// from it (commit followed by verify, with one read and one write of the
// state instead of two reads and one write). Blocks hold tokens of one set:
// the prefix's first, then the drafts'.
template <typename InT, typename OutT, int DK, int DV, int GATE, int TB, bool FUSED, bool STREAM>
__global__ __launch_bounds__((DV < kVerifyCols ? DV : kVerifyCols) * 4) void kda_spec_verify_cols(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const InT* __restrict__ g, const InT* __restrict__ beta, float* __restrict__ S,
    OutT* __restrict__ o, int64_t T, int64_t H, int64_t units, const InT* __restrict__ k1,
    const InT* __restrict__ v1, const InT* __restrict__ g1, const InT* __restrict__ beta1,
    const int32_t* __restrict__ accepted, int64_t T1) {
  constexpr int R = DK / 16;
  constexpr int CW = DV < kVerifyCols ? DV : kVerifyCols, NT = CW * 4, HALVES = DV / CW;
  // a block's token inputs: 16-byte vectors of q, k, g (TB x DK each) and of
  // this workgroup's v columns (TB x CW); thread t loads vectors t, t + NT, ...
  constexpr int VE = 16 / sizeof(InT);
  constexpr int NQ = TB * DK / VE, NVEC = 3 * NQ + TB * CW / VE, PER = (NVEC + NT - 1) / NT;
  static_assert(NQ % 64 == 0 && (TB * CW / VE) % 64 == 0, "input choice uniform per wavefront");
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  struct Block {
    u32x4v x[PER];
    InT b;
  };
  __shared__ __attribute__((aligned(16))) float s_q[TB][DK], s_k[TB][DK], s_e[TB][DK], s_v[TB][CW];
  __shared__ float s_b[TB];

  // XCD-aware numbering: workgroups are dealt to the 8 XCDs in turn, so the
  // HALVES workgroups of a unit take ids congruent mod 8 and share one L2
  // for their common inputs
  const int64_t bid = blockIdx.x;
  const int64_t unit = (bid / (8 * HALVES)) * 8 + bid % 8;
  const int half = static_cast<int>((bid / 8) % HALVES);
  if (unit >= units) return;  // uniform per workgroup; no barrier passed yet
  const int64_t n = unit / H, h = unit % H;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int rho = l >> 4, cq = l & 3;
  const int row0 = R * (l >> 2), lcol = 16 * w + 4 * cq;  // first row, first local column
  const int col = CW * half + lcol;                       // first column held
  const int locol = lcol + rho, ocol = col + rho;         // the column formed here

  // Tokens: ntok of the prefix (FUSED), then the T drafts; block b holds
  // prefix tokens [b TB, ..) for b < nc, else drafts [(b - nc) TB, ..).
  int64_t ntok = 0;
  if constexpr (FUSED) {
    const int64_t acc = accepted[n];
    ntok = acc < 0 ? 0 : (acc > T1 ? T1 : acc);
  }
  const int64_t nc = (ntok + TB - 1) / TB, nblocks = nc + (T + TB - 1) / TB;
  if (nblocks == 0) return;  // uniform per workgroup
  struct Where {
    bool pre;  // a block of the prefix
    int64_t t0;
    int nb;
  };
  auto where = [&](int64_t b) {
    Where x;
    x.pre = FUSED && b < nc;
    x.t0 = (x.pre ? b : b - nc) * TB;
    const int64_t left = (x.pre ? ntok : T) - x.t0;
    x.nb = static_cast<int>(left < TB ? left : TB);
    return x;
  };

  // Vector i of a block is vector r of input `which` (q, k, g, v: the
  // counts are multiples of 64, so the choice is uniform per wavefront; the
  // prefix has no q); fn gets the input's pointer, its LDS rows, the row
  // width in LDS, the input's row length and r.
  auto with_vec = [&](int i, bool pre, auto&& fn) __attribute__((always_inline)) {
    if (i < NQ) {
      if (!pre) fn(q, &s_q[0][0], DK, DK, i, false);
    } else if (i < 2 * NQ) {
      fn(pre ? k1 : k, &s_k[0][0], DK, DK, i - NQ, false);
    } else if (i < 3 * NQ) {
      fn(pre ? g1 : g, &s_e[0][0], DK, DK, i - 2 * NQ, true);
    } else if (i < NVEC) {
      fn((pre ? v1 : v) + CW * half, &s_v[0][0], CW, DV, i - 3 * NQ, false);
    }
  };
  auto load_block = [&](Block& x, const Where& wb) __attribute__((always_inline)) {
    const int64_t tn = wb.pre ? T1 : T;  // tokens per request in that set
    const size_t tok0 = static_cast<size_t>((n * tn + wb.t0) * H + h);  // token j: tok0 + j * H
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      with_vec(tid + e * NT, wb.pre, [&](const InT* base, float*, int width, int len, int r, bool) {
        const int j = r / (width / VE), c = (r % (width / VE)) * VE;
        if (j < wb.nb)
          x.x[e] = *reinterpret_cast<const u32x4v*>(base + (tok0 + static_cast<size_t>(j) * H) * len + c);
      });
    }
    if (tid < wb.nb) x.b = (wb.pre ? beta1 : beta)[tok0 + static_cast<size_t>(tid) * H];
  };
  // Stage: widen to fp32 (g to its decay factor e^gate) into the LDS rows.
  auto stage_block = [&](const Block& x, const Where& wb) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      with_vec(tid + e * NT, wb.pre, [&](const InT*, float* rows, int width, int, int r, bool decay) {
        const int j = r / (width / VE), c = (r % (width / VE)) * VE;
        if (j < wb.nb) {
          float f[VE];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            if constexpr (sizeof(InT) == 2) {  // bf16 pairs, low half first
              f[2 * m] = __uint_as_float(x.x[e][m] << 16);
              f[2 * m + 1] = __uint_as_float(x.x[e][m] & 0xffff0000u);
            } else {
              f[m] = __uint_as_float(x.x[e][m]);
            }
          }
          if (decay) {
#pragma unroll
            for (int m = 0; m < VE; ++m) f[m] = expf(gate_decay<GATE>(f[m]));
          }
          float* dst = rows + j * width + c;
#pragma unroll
          for (int m = 0; m < VE; m += 4)
            *reinterpret_cast<f32x4*>(dst + m) = f32x4{f[m], f[m + 1], f[m + 2], f[m + 3]};
        }
      });
    }
    if (tid < wb.nb) s_b[tid] = to_f32(x.b);
  };

  // inputs first: loads complete in order, so staging them waits only for them
  Block blk;
  load_block(blk, where(0));
  // The state: a 128-byte line holds 32 columns, which two wavefronts read
  // half each. Plain loads keep the line in the L2 for the second half;
  // loads with the streaming hint fetched about a quarter of the lines twice
  // (counters: 1.24x the algorithmic bytes), yet were faster for one or two
  // drafts (STREAM, chosen by the launcher).
  float* const Su = S + static_cast<size_t>(unit) * DK * DV + col;
  f32x4 s[R];
  if constexpr (STREAM) {
#pragma unroll
    for (int i = 0; i < R; ++i)
      s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Su + (row0 + i) * DV));
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) s[i] = *reinterpret_cast<const f32x4*>(Su + (row0 + i) * DV);
  }
  for (int64_t b = 0; b < nblocks; ++b) {
    const Where wb = where(b);
    if (b > 0) __syncthreads();  // the readers of the previous block are done
    stage_block(blk, wb);
    __syncthreads();
    if (b + 1 < nblocks) load_block(blk, where(b + 1));  // in flight while these tokens run
    if (FUSED && nc > 0 && b == nc) {
      // the accepted prefix is in: the new checkpoint, stored once the first
      // drafts are staged (stores issued earlier would hold up that wait,
      // which drains in issue order)
#pragma unroll
      for (int i = 0; i < R; ++i)
        __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Su + (row0 + i) * DV));
    }
    for (int j = 0; j < wb.nb; ++j) {
      // decay, then S^T k (and for a draft S^T q and q . k) of the lane's rows
      float r[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < R; i4 += 4) {
        const f32x4 e4 = *reinterpret_cast<const f32x4*>(&s_e[j][row0 + i4]);
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(&s_k[j][row0 + i4]);
        f32x4 q4 = zero4();
        if (!wb.pre) q4 = *reinterpret_cast<const f32x4*>(&s_q[j][row0 + i4]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int i = i4 + m;
          s[i] *= e4[m];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            r[c] += k4[m] * s[i][c];
            p[c] += q4[m] * s[i][c];
          }
          qk += q4[m] * k4[m];
        }
      }
      // row rho ends with the sums of column 4 cq + rho
      const float rs = sum_quads_of_row(swap_add32(swap_add16(r[0], r[1]), swap_add16(r[2], r[3])));
      const float u = s_b[j] * (s_v[j][locol] - rs);
      if (!wb.pre) {  // a draft: its output, from the state before its write
        const float ps = sum_quads_of_row(swap_add32(swap_add16(p[0], p[1]), swap_add16(p[2], p[3])));
        qk = swap_add16(qk, own_copy(qk));
        qk = sum_quads_of_row(swap_add32(qk, own_copy(qk)));
        if ((l & 12) == 0)  // one lane per column
          store_out(o, static_cast<size_t>((n * T + wb.t0 + j) * H + h) * DV + ocol, ps + qk * u);
      }
      // u of columns 4 cq + 0..3 to every row: rows {0,1} <- u0 / u1 pairs, ...
      const auto a = __builtin_amdgcn_permlane16_swap(fbits(u), fbits(own_copy(u)), false, false);
      const float ue = bitsf(a[0]), uo = bitsf(a[1]);  // u of rows 0, 2 / of rows 1, 3
      const auto bb = __builtin_amdgcn_permlane32_swap(fbits(ue), fbits(own_copy(ue)), false, false);
      const auto cc = __builtin_amdgcn_permlane32_swap(fbits(uo), fbits(own_copy(uo)), false, false);
      const f32x4 uc = {bitsf(bb[0]), bitsf(cc[0]), bitsf(bb[1]), bitsf(cc[1])};
#pragma unroll
      for (int i4 = 0; i4 < R; i4 += 4) {  // k read again: fewer live registers
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(&s_k[j][row0 + i4]);
#pragma unroll
        for (int m = 0; m < 4; ++m) s[i4 + m] += k4[m] * uc;
      }
    }
  }
  if (FUSED && nc > 0 && nblocks == nc) {  // no drafts (the launcher sends that case to the commit)
#pragma unroll
    for (int i = 0; i < R; ++i)
      __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Su + (row0 + i) * DV));
  }
}

// The column-slice kernel loads token inputs as 16-byte vectors; callers'
// pointers need only element alignment, so verify with other pointers takes
// the workgroup-per-unit form, and the fused call the two separate calls.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool verify_cols_aligned(const SpecArgs& a) {
  return aligned16(a.q) && aligned16(a.k) && aligned16(a.g) && aligned16(a.v);
}

enum SpecMode { kSpecVerify = 0, kSpecCommit = 1, kSpecFused = 2 };

// The column-slice kernel over whole groups of 8 units; false if the grid
// would exceed the launch limit (the caller then takes another form).
template <typename InT, typename OutT, int DK, int DV, int GATE, bool FUSED>
bool launch_cols(const SpecArgs& a, const SpecPrefix* pre, hipStream_t stream, hipError_t* err) {
  constexpr int CW = DV < kVerifyCols ? DV : kVerifyCols;
  const int64_t units = a.N * a.H;
  const int64_t grid = (units + 7) / 8 * 8 * (DV / CW);
  if (grid > 0x7fffffff) return false;
  // blocks of 16 tokens beyond 8 in either set; streaming state loads only
  // for a plain verify of one or two drafts (measured: 112 against 125 us at
  // one draft; plain loads are faster from four drafts on, and always fused)
  const int64_t tmax = FUSED && pre->T1 > a.T ? pre->T1 : a.T;
  auto kernel = tmax > 8  ? kda_spec_verify_cols<InT, OutT, DK, DV, GATE, 16, FUSED, false>
                : FUSED || a.T > 2 ? kda_spec_verify_cols<InT, OutT, DK, DV, GATE, 8, FUSED, false>
                                   : kda_spec_verify_cols<InT, OutT, DK, DV, GATE, 8, FUSED, !FUSED>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(grid)), dim3(CW * 4), 0, stream,
                     static_cast<const InT*>(a.q), static_cast<const InT*>(a.k),
                     static_cast<const InT*>(a.v), static_cast<const InT*>(a.g),
                     static_cast<const InT*>(a.beta), a.S, static_cast<OutT*>(a.o), a.T, a.H,
                     units, static_cast<const InT*>(FUSED ? pre->k1 : nullptr),
                     static_cast<const InT*>(FUSED ? pre->v1 : nullptr),
                     static_cast<const InT*>(FUSED ? pre->g1 : nullptr),
                     static_cast<const InT*>(FUSED ? pre->beta1 : nullptr),
                     FUSED ? pre->accepted : nullptr, FUSED ? pre->T1 : int64_t{0});
  *err = hipGetLastError();
  return true;
}

template <typename InT, typename OutT, int DK, int DV, int GATE, int MODE>
hipError_t launch_typed(const SpecArgs& a, const SpecPrefix* pre, hipStream_t stream) {
  const int64_t units = a.N * a.H;
  hipError_t err = hipSuccess;
  if constexpr (MODE == kSpecFused) {
    if (verify_cols_aligned(a) && aligned16(pre->k1) && aligned16(pre->g1) && aligned16(pre->v1) &&
        launch_cols<InT, OutT, DK, DV, GATE, true>(a, pre, stream, &err))
      return err;
    // element-aligned inputs: the commit, then the verify
    SpecArgs c = a;
    c.q = nullptr;
    c.k = pre->k1;
    c.v = pre->v1;
    c.g = pre->g1;
    c.beta = pre->beta1;
    c.o = nullptr;
    c.accepted = pre->accepted;
    c.T = pre->T1;
    err = launch_typed<InT, float, DK, DV, GATE, kSpecCommit>(c, nullptr, stream);
    if (err != hipSuccess) return err;
    return launch_typed<InT, OutT, DK, DV, GATE, kSpecVerify>(a, nullptr, stream);
  } else {
    constexpr bool COMMIT = MODE == kSpecCommit;
    if (!COMMIT && verify_cols_aligned(a) &&
        launch_cols<InT, OutT, DK, DV, GATE, false>(a, nullptr, stream, &err))
      return err;
    // commit: persistent workgroups over the units; verify (inputs not 16-byte
    // aligned): one per unit
    const int64_t grid = COMMIT && units > kCommitGrid ? kCommitGrid : units;
    hipLaunchKernelGGL((kda_spec_kernel<InT, OutT, DK, DV, GATE, COMMIT>),
                       dim3(static_cast<uint32_t>(grid)), dim3(spec_threads<COMMIT>()), 0, stream,
                       static_cast<const InT*>(a.q), static_cast<const InT*>(a.k),
                       static_cast<const InT*>(a.v), static_cast<const InT*>(a.g),
                       static_cast<const InT*>(a.beta), a.S, static_cast<OutT*>(a.o), a.accepted,
                       a.T, a.H, units);
    return hipGetLastError();
  }
}

template <typename InT, typename OutT, int DK, int DV, int MODE>
hipError_t launch_gate(const SpecArgs& a, const SpecPrefix* pre, hipStream_t s) {
  return a.gate == kGateSigmoid ? launch_typed<InT, OutT, DK, DV, kGateSigmoid, MODE>(a, pre, s)
                                : launch_typed<InT, OutT, DK, DV, kGateLogDecay, MODE>(a, pre, s);
}

template <typename InT, typename OutT, int MODE>
hipError_t launch_shape(const SpecArgs& a, const SpecPrefix* pre, hipStream_t s) {
  if (a.dk == 64)
    return a.dv == 64 ? launch_gate<InT, OutT, 64, 64, MODE>(a, pre, s)
                      : launch_gate<InT, OutT, 64, 128, MODE>(a, pre, s);
  return a.dv == 64 ? launch_gate<InT, OutT, 128, 64, MODE>(a, pre, s)
                    : launch_gate<InT, OutT, 128, 128, MODE>(a, pre, s);
}

template <int MODE>
hipError_t launch_out(const SpecArgs& a, const SpecPrefix* pre, hipStream_t stream) {
  const bool in32 = a.in_dtype == 0, out32 = a.out_dtype == 0;
  if (in32)
    return out32 ? launch_shape<float, float, MODE>(a, pre, stream)
                 : launch_shape<float, uint16_t, MODE>(a, pre, stream);
  return out32 ? launch_shape<uint16_t, float, MODE>(a, pre, stream)
               : launch_shape<uint16_t, uint16_t, MODE>(a, pre, stream);
}

}  // namespace

hipError_t launch_spec(const SpecArgs& a, bool commit, hipStream_t stream) {
  if (a.N * a.H == 0 || a.T == 0) return hipSuccess;
  if (commit)  // no output: the output type is immaterial
    return a.in_dtype == 0 ? launch_shape<float, float, kSpecCommit>(a, nullptr, stream)
                           : launch_shape<uint16_t, float, kSpecCommit>(a, nullptr, stream);
  return launch_out<kSpecVerify>(a, nullptr, stream);
}

hipError_t launch_spec_commit_verify(const SpecArgs& drafts, const SpecPrefix& pre,
                                     hipStream_t stream) {
  if (drafts.N * drafts.H == 0) return hipSuccess;
  if (pre.T1 == 0) return launch_spec(drafts, false, stream);
  if (drafts.T == 0) {  // the commit alone
    SpecArgs c = drafts;
    c.q = nullptr;
    c.k = pre.k1;
    c.v = pre.v1;
    c.g = pre.g1;
    c.beta = pre.beta1;
    c.o = nullptr;
    c.accepted = pre.accepted;
    c.T = pre.T1;
    return launch_spec(c, true, stream);
  }
  return launch_out<kSpecFused>(drafts, &pre, stream);
}

}  // namespace kda
