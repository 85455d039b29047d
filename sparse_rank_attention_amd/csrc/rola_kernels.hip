// rola_kernels.hip -- gfx950 (CDNA4) kernels of librola.
//
// RoLA attention (pages: "SparkDiffusion: 265x Faster Video Generation on
// Consumer GPUs via Sparse Attention & Distillation", section "RoLA:
// Preserving Global Context at Extreme Sparsity"): a block-sparse softmax
// branch over the highest-energy query-key blocks plus a rotary-positioned
// low-rank linear branch; the output is their sum.
//
// Kernels, in launch order:
//   k_setup        rotary cos/sin table, bf16 transposed projections
//   k_pass1        one streaming pass over the token tensors: block pooling
//                  of Q and K (fixed fp32 tree order), low-rank state partials
//                  from K and V (MFMA), and the transposed V tiles the sparse
//                  kernel reads
//   k_state_reduce fixed-order sum of the state partials
//   k_scores       pooled block scores, sequential fp32 fma chain (VALU)
//   k_topk         per-row radix select of the kept key blocks (one wave/row)
//   k_attn         block-sparse flash attention on bf16 MFMA with online
//                  softmax in fp32, fused low-rank apply and merge
//
// MFMA conventions (v_mfma_f32_32x32x16_bf16, wave64): lane l, g = l/32.
//   A operand: row l%32, 8 consecutive k values of group g;
//   B operand: column l%32, 8 consecutive k values of group g;
//   C/D: 16 floats, column l%32, row 8*(i/4) + 4*g + i%4 for element i.
// Attention is computed transposed (S^T = K Q^T, O^T = V^T P^T) so that one
// lane owns one query column throughout: its softmax statistics are lane
// scalars, and the S^T accumulator is directly the B operand of the PV step
// provided the key order inside every 16-key group is permuted as
// [0-3, 8-11, 4-7, 12-15] in the transposed V tile.  The same permutation is
// used for the rank index of the low-rank state and for tokens in the state
// contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rola_internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

namespace rola {

static __device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
static __device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
static __device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

static __device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
static __device__ __forceinline__ u32x4 as_u32x4(bf16x8 b) { return __builtin_bit_cast(u32x4, b); }

// Physical position of a key (or rank index) inside a 16-group of the
// transposed tiles: keys [0-3, 8-11, 4-7, 12-15] are stored at 0..15.
static __device__ __forceinline__ int perm16_key_of_pos(int p) {
  const int w = p & 15;
  const int k = (w < 4) ? w : (w < 8) ? w + 4 : (w < 12) ? w - 4 : w;
  return (p & ~15) | k;
}

static __device__ __forceinline__ float phi(float u) { return u > 0.0f ? u + 1.0f : __expf(u); }

static __device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

static __device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

static __device__ __forceinline__ void lds_dma16(const void *gsrc, void *lds_dst) {
  __builtin_amdgcn_global_load_lds((const GLOBAL_AS void *)gsrc, (LDS_AS void *)lds_dst, 16, 0, 0);
}

// Rotary tables: tab holds (cos, sin) per axis, position and pair; the t,
// h and w axes own dims [0, off1), [off1, off2), [off2, D).
using RopeArgsDev = RopeArgsHost;

static __device__ __forceinline__ void token_pos(int64_t n, const RopeArgsDev &ra, int &pt, int &ph,
                                                 int &pw) {
  const int hw = ra.grid_h * ra.grid_w;
  pt = (int)(n / hw);
  const int rem = (int)(n - (int64_t)pt * hw);
  ph = rem / ra.grid_w;
  pw = rem - ph * ra.grid_w;
}

static __device__ __forceinline__ float2 rope_cs(int d, int pt, int ph, int pw, const RopeArgsDev &ra) {
  int idx;
  if (d < ra.off1)
    idx = pt * ra.half0 + (d >> 1);
  else if (d < ra.off2)
    idx = ra.tab1 + ph * ra.half1 + ((d - ra.off1) >> 1);
  else
    idx = ra.tab2 + pw * ra.half2 + ((d - ra.off2) >> 1);
  return ra.tab[idx];
}

// Rotate 8 consecutive dims (4 pairs) starting at d0 and round to bf16.
static __device__ __forceinline__ bf16x8 rope8(bf16x8 x, int d0, int pt, int ph, int pw,
                                               const RopeArgsDev &ra) {
  const u32x4 u = as_u32x4(x);
  bf16x8 y;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float x0 = bflo(u[p]), x1 = bfhi(u[p]);
    const float2 cs = rope_cs(d0 + 2 * p, pt, ph, pw, ra);
    y[2 * p] = (__bf16)(x0 * cs.x - x1 * cs.y);
    y[2 * p + 1] = (__bf16)(x0 * cs.y + x1 * cs.x);
  }
  return y;
}

// ---------------------------------------------------------------- k_setup
__global__ void k_setup(const float *__restrict__ wq, const float *__restrict__ wk, int D, int rank,
                        uint16_t *__restrict__ wqT, uint16_t *__restrict__ wkT, float2 *tab,
                        int tab_total, int g0, int g1, int h0, int h1, int h2, double theta) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  // transposed bf16 projections [32][D], rows >= rank zero
  if (tid < 32 * D) {
    const int r = tid / D, d = tid % D;
    float a = 0.0f, b = 0.0f;
    if (r < rank) {
      a = wq[d * rank + r];
      b = wk[d * rank + r];
    }
    const __bf16 ab = (__bf16)a, bb = (__bf16)b;
    wqT[tid] = __builtin_bit_cast(uint16_t, ab);
    wkT[tid] = __builtin_bit_cast(uint16_t, bb);
  }
  // rotary table: axis a, position pos, pair p -> (cos, sin) of pos * theta^(-2p/d_a)
  if (tid < tab_total) {
    int a, pos, p, da;
    const int n0 = g0 * h0, n1 = g1 * h1;
    if (tid < n0) {
      a = 0; pos = tid / h0; p = tid % h0; da = 2 * h0;
    } else if (tid < n0 + n1) {
      a = 1; pos = (tid - n0) / h1; p = (tid - n0) % h1; da = 2 * h1;
    } else {
      a = 2; pos = (tid - n0 - n1) / h2; p = (tid - n0 - n1) % h2; da = 2 * h2;
    }
    (void)a;
    const double ang = (double)pos * pow(theta, -2.0 * p / (double)da);
    tab[tid] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

// ---------------------------------------------------------------- k_pass1
// Grid (nchunks, B*H), 256 threads.  Each workgroup walks `cpc` consecutive
// 64-token blocks of one (batch, head).
//   POOL : waves 0 and 1 pool Q and K (fixed tree order) into Qp, Kp.
//   STATE: waves 2 and 3 form b = phi(Wk^T R(k)) for the block (MFMA) and
//          accumulate S^T += V^T b (MFMA) and z += b; partials per workgroup.
//   VT   : the transposed, key-permuted, chunk-swizzled V tile is written to
//          the workspace in the exact LDS image the attention kernel loads.
template <int D, bool POOL, bool STATE, bool VT>
__global__ __launch_bounds__(256) void k_pass1(Pass1Args args) {
  constexpr int CH = D / 8;  // 16-byte chunks per token row
  __shared__ __attribute__((aligned(16))) uint16_t sQ[POOL ? 64 * D : 1];
  __shared__ __attribute__((aligned(16))) uint16_t sK[(POOL || STATE) ? 64 * D : 1];
  __shared__ __attribute__((aligned(16))) uint16_t sV[(STATE || VT) ? 64 * D : 1];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[(STATE || VT) ? 64 * D : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int bh = blockIdx.y;
  const int b = bh / args.heads, h = bh % args.heads;
  const int64_t base = (int64_t)b * args.stride_b + (int64_t)h * args.stride_h;
  const uint16_t *Q = args.q + base, *K = args.k + base, *V = args.v + base;
  const int c0 = blockIdx.x * args.cpc;
  const int c1 = min(args.nb, c0 + args.cpc);

  const RopeArgsDev ra = args.rope;
  // state accumulators: wave 2 owns d-tiles [0, D/64), wave 3 [D/64, D/32)
  constexpr int DT = D / 64;
  f32x16 sacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) sacc[i] = f32x16{};
  float zacc = 0.0f;
  bf16x8 wkreg[D / 16];
  if (STATE && wave >= 2) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      wkreg[s] = *(const bf16x8 *)(args.wkT + (lane & 31) * D + 16 * s + 8 * g);
  }

  for (int c = c0; c < c1; ++c) {
    const int valid = min(64, (int)(args.n_tokens - (int64_t)c * 64));
    // ---- stage tiles in LDS (plain 16-byte loads; rows >= valid are zeroed)
    for (int cidx = tid; cidx < 64 * CH; cidx += 256) {
      const int row = cidx / CH, col = cidx % CH;
      const int64_t goff = ((int64_t)c * 64 + row) * args.stride_n + col * 8;
      const bool ok = row < valid;
      if (POOL) {
        u32x4 x = ok ? *(const u32x4 *)(Q + goff) : u32x4{0, 0, 0, 0};
        *(u32x4 *)(sQ + row * D + col * 8) = x;
      }
      if (POOL || STATE) {
        u32x4 x = ok ? *(const u32x4 *)(K + goff) : u32x4{0, 0, 0, 0};
        *(u32x4 *)(sK + row * D + ((col ^ (row & 7)) * 8)) = x;
      }
      if (STATE || VT) {
        u32x4 x = ok ? *(const u32x4 *)(V + goff) : u32x4{0, 0, 0, 0};
        *(u32x4 *)(sV + row * D + col * 8) = x;
      }
    }
    __syncthreads();

    // ---- transposed V tile: row d, 64 keys permuted per 16-group, chunks swizzled by d&7
    if (STATE || VT) {
      // task = (d pair, logical chunk): 8 keys of two dims
      for (int task = tid; task < (D / 2) * 8; task += 256) {
        const int dp = task % (D / 2), lc = task / (D / 2);
        const int d = 2 * dp;
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = perm16_key_of_pos(lc * 8 + e);
          w[e] = *(const uint32_t *)(sV + key * D + d);
        }
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = (w[2 * e] & 0xffffu) | (w[2 * e + 1] << 16);
          hi[e] = (w[2 * e] >> 16) | (w[2 * e + 1] & 0xffff0000u);
        }
        *(u32x4 *)(sVt + d * 64 + ((lc ^ (d & 7)) * 8)) = lo;
        *(u32x4 *)(sVt + (d + 1) * 64 + ((lc ^ ((d + 1) & 7)) * 8)) = hi;
      }
      __syncthreads();
      if (VT) {
        uint16_t *dst = args.vt + ((int64_t)bh * args.nb + c) * (64 * D);
        for (int cidx = tid; cidx < 64 * CH; cidx += 256)
          *(u32x4 *)(dst + cidx * 8) = *(const u32x4 *)(sVt + cidx * 8);
      }
    }

    // ---- pooling: wave 0 -> Q, wave 1 -> K; lane owns dims 2*lane, 2*lane+1
    if (POOL && wave < 2 && lane < D / 2) {
      const uint16_t *tile = wave == 0 ? sQ : sK;
      const int word = lane;
      float lo[32], hi[32];
#pragma unroll
      for (int s = 0; s < 32; ++s) {
        const int off = wave == 0 ? s * D + 2 * word
                                  : s * D + ((((word >> 2) ^ (s & 7)) << 3) | ((word & 3) << 1));
        const uint32_t x = *(const uint32_t *)(tile + off);
        lo[s] = bflo(x);
        hi[s] = bfhi(x);
      }
#pragma unroll
      for (int s = 32; s < 64; ++s) {
        const int off = wave == 0 ? s * D + 2 * word
                                  : s * D + ((((word >> 2) ^ (s & 7)) << 3) | ((word & 3) << 1));
        const uint32_t x = *(const uint32_t *)(tile + off);
        lo[s - 32] = lo[s - 32] + bflo(x);
        hi[s - 32] = hi[s - 32] + bfhi(x);
      }
#pragma unroll
      for (int stride = 16; stride >= 1; stride >>= 1) {
#pragma unroll
        for (int i = 0; i < stride; ++i) {
          lo[i] = lo[i] + lo[i + stride];
          hi[i] = hi[i] + hi[i + stride];
        }
      }
      const float inv = valid == 64 ? 0.015625f : args.inv_tail;
      float *dst = (wave == 0 ? args.qp : args.kp) + ((int64_t)bh * args.nb + c) * D + 2 * word;
      *(float2 *)dst = make_float2(lo[0] * inv, hi[0] * inv);
    }

    // ---- low-rank state: waves 2 and 3
    if (STATE && wave >= 2) {
      // b tile [64 tokens x 32 r]: A = R(K) (rows tokens), B = Wk^T (cols r)
      f32x16 bacc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bacc[tt] = f32x16{};
        const int row = 32 * tt + (lane & 31);
        int pt, ph, pw;  // padded rows take the last valid position (their b is masked)
        token_pos(min((int64_t)c * 64 + row, args.n_tokens - 1), ra, pt, ph, pw);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const int lc = 2 * s + g;
          bf16x8 kx = *(const bf16x8 *)(sK + row * D + ((lc ^ (row & 7)) * 8));
          kx = rope8(kx, 16 * s + 8 * g, pt, ph, pw, ra);
          bacc[tt] = mfma_bf16(kx, wkreg[s], bacc[tt]);
        }
      }
      // phi, mask invalid tokens and rank padding, accumulate z, pack as B operand
      const bool rok = (lane & 31) < args.rank;
      bf16x8 bop[4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = 32 * tt + 8 * (i >> 2) + 4 * g + (i & 3);
          float f = phi(bacc[tt][i]);
          f = (rok && tok < valid) ? f : 0.0f;
          zacc += f;
          bop[2 * tt + (i >> 3)][i & 7] = (__bf16)f;
        }
      }
      // S^T[d][r] += sum_tok Vt[d][tok] * b[tok][r]
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int dt = (wave - 2) * DT + t;
        const int d = 32 * dt + (lane & 31);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int lc = 2 * s + g;
          const bf16x8 va = *(const bf16x8 *)(sVt + d * 64 + ((lc ^ (d & 7)) * 8));
          sacc[t] = mfma_bf16(va, bop[s], sacc[t]);
        }
      }
    }
    __syncthreads();
  }

  if (STATE && wave >= 2) {
    float *part = args.state_part + ((int64_t)bh * gridDim.x + blockIdx.x) * (D * 32 + 32);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int dt = (wave - 2) * DT + t;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * dt + 8 * (i >> 2) + 4 * g + (i & 3);
        part[d * 32 + (lane & 31)] = sacc[t][i];
      }
    }
    const float zt = zacc + shfl_xor32(zacc);
    if (wave == 2 && lane < 32) part[D * 32 + lane] = zt;
  }
}

// ------------------------------------------------------------ k_state_reduce
// One workgroup per (batch, head): fixed-order sum over the chunk partials.
// Writes St (bf16 [D][32], rank index permuted per 16-group, the A operand
// layout of the apply step) and z (fp32 [32]).  Rank columns >= rank are 0.
__global__ __launch_bounds__(256) void k_state_reduce(const float *__restrict__ part, int nchunks,
                                                      int D, int rank, uint16_t *__restrict__ st,
                                                      float *__restrict__ z) {
  const int bh = blockIdx.x;
  const int stride = D * 32 + 32;
  const float *p = part + (int64_t)bh * nchunks * stride;
  for (int idx = threadIdx.x; idx < stride; idx += blockDim.x) {
    float acc = 0.0f;
    for (int c = 0; c < nchunks; ++c) acc += p[(int64_t)c * stride + idx];
    if (idx < D * 32) {
      const int d = idx / 32, r = idx % 32;
      // position of rank r in the permuted row
      int pos = 0;
      {
        const int w = r & 15;
        const int pw = (w < 4) ? w : (w < 8) ? w + 4 : (w < 12) ? w - 4 : w;
        pos = (r & ~15) | pw;
      }
      const __bf16 v = (__bf16)(r < rank ? acc : 0.0f);
      st[(int64_t)bh * D * 32 + d * 32 + pos] = __builtin_bit_cast(uint16_t, v);
    } else {
      const int r = idx - D * 32;
      z[(int64_t)bh * 32 + r] = r < rank ? acc : 0.0f;
    }
  }
}

// --------------------------------------------------------------- k_scores
// s[bh][i][j] = sequential fma chain over d of Qp[i][d] * Kp[j][d] from +0.0.
// Lane = key block j (its Kp row in registers), rows i wave-uniform.
template <int D>
__global__ __launch_bounds__(256) void k_scores(const float *__restrict__ qp,
                                                const float *__restrict__ kp, float *__restrict__ s,
                                                int nb, int rows_per_wg) {
#pragma clang fp contract(off)
  const int bh = blockIdx.z;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int jl = j < nb ? j : nb - 1;
  const float *kr = kp + ((int64_t)bh * nb + jl) * D;
  float kreg[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const f32x4 x = *(const f32x4 *)(kr + d);
    kreg[d] = x[0]; kreg[d + 1] = x[1]; kreg[d + 2] = x[2]; kreg[d + 3] = x[3];
  }
  const int i0 = blockIdx.y * rows_per_wg;
  const int i1 = min(nb, i0 + rows_per_wg);
  for (int i = i0; i < i1; ++i) {
    const float *qr = qp + ((int64_t)bh * nb + i) * D;
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qr[d], kreg[d], acc);
    if (j < nb) s[((int64_t)bh * nb + i) * nb + j] = acc;
  }
}

// ----------------------------------------------------------------- k_topk
// One wave per score row: order-preserving uint32 keys (-0.0 folded into
// +0.0), bitwise search for the kb-th largest key T, then emit, in ascending
// index order, every j with key > T and the lowest-index ties key == T.
static __device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int PER>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ s, int32_t *__restrict__ map,
                                              int nb, int kb, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float *sr = s + row * nb;
  uint32_t key[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int j = m * 64 + lane;
    key[m] = j < nb ? order_key(sr[j]) : 0u;  // real keys are >= 0x007fffff
  }
  uint32_t prefix = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) cnt += __popcll(__ballot(key[m] >= cand));
    if (cnt >= kb) prefix = cand;
  }
  const uint32_t T = prefix;
  int greater = 0;
#pragma unroll
  for (int m = 0; m < PER; ++m) greater += __popcll(__ballot(key[m] > T));
  const int take_eq = kb - greater;
  int out = 0, ties = 0;
  int32_t *mr = map + row * kb;
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const uint64_t eqm = __ballot(key[m] == T);
    const uint32_t below_eq =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(eqm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eqm, 0u));
    const bool sel = key[m] > T || (key[m] == T && ties + (int)below_eq < take_eq);
    const uint64_t selm = __ballot(sel);
    const uint32_t below_sel = __builtin_amdgcn_mbcnt_hi((uint32_t)(selm >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)selm, 0u));
    if (sel) mr[out + (int)below_sel] = m * 64 + lane;
    out += __popcll(selm);
    ties += __popcll(eqm);
  }
}

// ----------------------------------------------------------------- k_attn
// One workgroup (2 waves) per (batch, head, query block); wave w owns query
// rows 32w..32w+31 of the block, one query per lane column.  K and V^T tiles
// of each kept key block are copied global->LDS directly (16 B per lane).
template <int D, bool SPARSE, bool LOWRANK, bool ACCUM, bool OUTF32>
__global__ __launch_bounds__(128) void k_attn(AttnArgs args) {
  constexpr int CH = D / 8;
  constexpr int NS = D / 16;  // k-steps over head_dim
  constexpr int DT = D / 32;  // output d-tiles
  __shared__ __attribute__((aligned(1024))) uint16_t sK[SPARSE ? 64 * D : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[SPARSE ? 64 * D : 8];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  // XCD-aware order: consecutive workgroups of one XCD take consecutive
  // query blocks of one head, so their K/V gathers share that XCD's L2.
  const int64_t L = blockIdx.x;
  const int64_t tile = (L % 8) * args.tiles_per_xcd + (L / 8);
  if (tile >= args.tiles || (L / 8) >= args.tiles_per_xcd) return;
  const int bh = (int)(tile / args.nb);
  const int qb = (int)(tile % args.nb);
  const int b = bh / args.heads, h = bh % args.heads;
  const int64_t base = (int64_t)b * args.stride_b + (int64_t)h * args.stride_h;
  const int64_t n = (int64_t)qb * 64 + 32 * wave + (lane & 31);  // this lane's query token

  bf16x8 qreg[NS];
  {
    const uint16_t *qrow = args.q + base + n * args.stride_n;
#pragma unroll
    for (int s = 0; s < NS; ++s) qreg[s] = *(const bf16x8 *)(qrow + 16 * s + 8 * g);
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  if (SPARSE) {
    const int32_t *mrow = args.map + ((int64_t)bh * args.nb + qb) * args.kb;
    const uint16_t *Kb = args.k + base;
    const uint16_t *Vtb = args.vt + (int64_t)bh * args.nb * (64 * D);
    const float c = args.scale_log2e;
    const int tid = threadIdx.x;
    for (int t = 0; t < args.kb; ++t) {
      // ids outside [0, nb) (a malformed caller map) are clamped: wrong output, no stray reads
      const int j = min(max(mrow[t], 0), args.nb - 1);
      // ---- copy K_j (chunk-swizzled rows) and V^T_j (already in LDS image order)
#pragma unroll
      for (int it = 0; it < (64 * CH) / 128; ++it) {
        const int cidx = it * 128 + tid;
        const int row = cidx / CH, pc = cidx % CH;
        const int lc = pc ^ (row & 7);
        lds_dma16(Kb + ((int64_t)j * 64 + row) * args.stride_n + lc * 8,
                  sK + (it * 128 + wave * 64) * 8);
        lds_dma16(Vtb + (int64_t)j * (64 * D) + cidx * 8, sV + (it * 128 + wave * 64) * 8);
      }
      __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0): both tiles landed in LDS
      __syncthreads();

      // ---- S^T = K Q^T (two 32-key tiles)
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sacc[kt] = f32x16{};
        const int row = 32 * kt + (lane & 31);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int lc = 2 * s + g;
          const bf16x8 ka = *(const bf16x8 *)(sK + row * D + ((lc ^ (row & 7)) * 8));
          sacc[kt] = mfma_bf16(ka, qreg[s], sacc[kt]);
        }
      }
      // ---- online softmax (base 2); keys >= N masked in the tail block
      const bool tail = (int64_t)(j + 1) * 64 > args.n_tokens;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = sacc[kt][i] * c;
          if (tail) {
            const int64_t key = (int64_t)j * 64 + 32 * kt + 8 * (i >> 2) + 4 * g + (i & 3);
            x = key < args.n_tokens ? x : -INFINITY;
          }
          sacc[kt][i] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, shfl_xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.0f;
      bf16x8 pop[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2f(sacc[kt][i] - m_new);
          psum += p;
          pop[2 * kt + (i >> 3)][i & 7] = (__bf16)p;
        }
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + (lane & 31);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int lc = 2 * s + g;
          const bf16x8 va = *(const bf16x8 *)(sV + d * 64 + ((lc ^ (d & 7)) * 8));
          oacc[dt] = mfma_bf16(va, pop[s], oacc[dt]);
        }
      }
      __syncthreads();  // all reads of sK/sV done before the next copy
    }
    const float l_tot = l_run + shfl_xor32(l_run);
    const float inv_l = args.kb > 0 ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= inv_l;
  }

  if (LOWRANK) {
    // a^T = Wq^T R(q): A = Wq^T (rows r), B = rotated Q (cols query)
    int pt, ph, pw;  // padded rows take the last valid position (they are written as 0)
    token_pos(n < args.n_tokens ? n : args.n_tokens - 1, args.rope, pt, ph, pw);
    f32x16 aacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 qr = rope8(qreg[s], 16 * s + 8 * g, pt, ph, pw, args.rope);
      const bf16x8 wa = *(const bf16x8 *)(args.wqT + (lane & 31) * D + 16 * s + 8 * g);
      aacc = mfma_bf16(wa, qr, aacc);
    }
    const float *zb = args.z + (int64_t)bh * 32;
    float den = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * g + (i & 3);
      const float a = r < args.rank ? phi(aacc[i]) : 0.0f;
      aacc[i] = a;
      den += a * zb[r];
    }
    den += shfl_xor32(den);
    const float inv_den = 1.0f / den;
    bf16x8 aop[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) aop[i >> 3][i & 7] = (__bf16)(aacc[i] * inv_den);
    const uint16_t *stb = args.st + (int64_t)bh * D * 32;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + (lane & 31);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 sa = *(const bf16x8 *)(stb + d * 32 + 16 * s + 8 * g);
        oacc[dt] = mfma_bf16(sa, aop[s], oacc[dt]);
      }
    }
  }

  // ---- write O row n: lane holds dims 32*dt + 8*q4 + 4*g + 0..3
  const bool valid = n < args.n_tokens;
  if (OUTF32) {
    float *orow = (float *)args.out + base + n * args.stride_n;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float *p = orow + 32 * dt + 8 * q4 + 4 * g;
        f32x4 v = {oacc[dt][4 * q4], oacc[dt][4 * q4 + 1], oacc[dt][4 * q4 + 2], oacc[dt][4 * q4 + 3]};
        if (ACCUM) v += *(const f32x4 *)p;
        if (!valid) v = f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4 *)p = v;
      }
    }
  } else {
    uint16_t *orow = (uint16_t *)args.out + base + n * args.stride_n;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint16_t *p = orow + 32 * dt + 8 * q4 + 4 * g;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[dt][4 * q4 + e];
        if (ACCUM) {
          const uint2 old = *(const uint2 *)p;
          v[0] += bflo(old.x); v[1] += bfhi(old.x);
          v[2] += bflo(old.y); v[3] += bfhi(old.y);
        }
        uint2 o;
        const __bf16 b0 = (__bf16)v[0], b1 = (__bf16)v[1], b2 = (__bf16)v[2], b3 = (__bf16)v[3];
        o.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        o.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        if (!valid) o = make_uint2(0u, 0u);
        *(uint2 *)p = o;
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
void launch_setup(const SetupArgs &a, hipStream_t st) {
  const int total = (32 * a.D > a.tab_total) ? 32 * a.D : a.tab_total;
  hipLaunchKernelGGL(k_setup, dim3((total + 255) / 256), dim3(256), 0, st, a.wq, a.wk, a.D, a.rank,
                     a.wqT, a.wkT, a.tab, a.tab_total, a.g0, a.g1, a.h0, a.h1, a.h2, a.theta);
}

template <int D>
static void pass1_d(const Pass1Args &a, int nchunks, int bh, bool pool, bool state, bool vt,
                    hipStream_t st) {
  dim3 grid(nchunks, bh), block(256);
  if (pool && state && vt)
    hipLaunchKernelGGL((k_pass1<D, true, true, true>), grid, block, 0, st, a);
  else if (pool && !state && !vt)
    hipLaunchKernelGGL((k_pass1<D, true, false, false>), grid, block, 0, st, a);
  else if (!pool && !state && vt)
    hipLaunchKernelGGL((k_pass1<D, false, false, true>), grid, block, 0, st, a);
  else if (!pool && state && !vt)
    hipLaunchKernelGGL((k_pass1<D, false, true, false>), grid, block, 0, st, a);
}

void launch_pass1(const Pass1Args &a, int D, int nchunks, int bh, bool pool, bool state, bool vt,
                  hipStream_t st) {
  if (D == 64) pass1_d<64>(a, nchunks, bh, pool, state, vt, st);
  else pass1_d<128>(a, nchunks, bh, pool, state, vt, st);
}

void launch_state_reduce(const float *part, int nchunks, int D, int rank, int bh, uint16_t *st_out,
                         float *z, hipStream_t st) {
  hipLaunchKernelGGL(k_state_reduce, dim3(bh), dim3(256), 0, st, part, nchunks, D, rank, st_out, z);
}

void launch_scores(const float *qp, const float *kp, float *s, int nb, int D, int bh,
                   hipStream_t st) {
  const int rows = 64;
  dim3 grid((nb + 255) / 256, (nb + rows - 1) / rows, bh);
  if (D == 64) hipLaunchKernelGGL(k_scores<64>, grid, dim3(256), 0, st, qp, kp, s, nb, rows);
  else hipLaunchKernelGGL(k_scores<128>, grid, dim3(256), 0, st, qp, kp, s, nb, rows);
}

void launch_topk(const float *s, int32_t *map, int nb, int kb, int64_t rows, hipStream_t st) {
  const int per = (nb + 63) / 64;
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
#define ROLA_TOPK(P) hipLaunchKernelGGL(k_topk<P>, grid, block, 0, st, s, map, nb, kb, rows)
  if (per <= 2) ROLA_TOPK(2);
  else if (per <= 4) ROLA_TOPK(4);
  else if (per <= 8) ROLA_TOPK(8);
  else if (per <= 12) ROLA_TOPK(12);
  else if (per <= 16) ROLA_TOPK(16);
  else if (per <= 20) ROLA_TOPK(20);
  else if (per <= 24) ROLA_TOPK(24);
  else if (per <= 32) ROLA_TOPK(32);
  else if (per <= 48) ROLA_TOPK(48);
  else ROLA_TOPK(64);
#undef ROLA_TOPK
}

template <int D, bool SPARSE, bool LOWRANK>
static void attn_d2(const AttnArgs &a, bool accum, bool outf32, hipStream_t st) {
  dim3 grid((unsigned)(8 * a.tiles_per_xcd)), block(128);
  if (accum) {
    if (outf32) hipLaunchKernelGGL((k_attn<D, SPARSE, LOWRANK, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn<D, SPARSE, LOWRANK, true, false>), grid, block, 0, st, a);
  } else {
    if (outf32) hipLaunchKernelGGL((k_attn<D, SPARSE, LOWRANK, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn<D, SPARSE, LOWRANK, false, false>), grid, block, 0, st, a);
  }
}

template <int D>
static void attn_d(const AttnArgs &a, bool sparse, bool lowrank, bool accum, bool outf32,
                   hipStream_t st) {
  if (sparse && lowrank) attn_d2<D, true, true>(a, accum, outf32, st);
  else if (sparse) attn_d2<D, true, false>(a, accum, outf32, st);
  else attn_d2<D, false, true>(a, accum, outf32, st);
}

void launch_attn(const AttnArgs &a, int D, bool sparse, bool lowrank, bool accum, bool outf32,
                 hipStream_t st) {
  if (D == 64) attn_d<64>(a, sparse, lowrank, accum, outf32, st);
  else attn_d<128>(a, sparse, lowrank, accum, outf32, st);
}

}  // namespace rola
