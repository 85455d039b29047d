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
//                  of Q and K (fixed fp32 tree order) and low-rank state
//                  partials from K and V (MFMA)
//   k_blk_partial  (complement scope) block-range sums of the per-block states
//   k_state_reduce fixed-order sum of the state partials
//   k_complement   (complement scope) per query block: global state minus
//                  the states of its kept key blocks
//   k_scores       pooled block scores, sequential fp32 fma chain (VALU)
//   k_topk         per-row radix select of the kept key blocks (one wave/row)
//   k_order        per head: query blocks ordered by similarity of their maps
//   k_group        greedy grouping of similar maps inside windows of that order
//   k_union        per group of query blocks: merged list of kept key blocks
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
// provided the V^T operand lists the keys of every 16-key step in the order
// [0-3, 8-11] (lanes 0-31) and [4-7, 12-15] (lanes 32-63); the transposing
// LDS read (ds_read_b64_tr_b16) produces exactly that from a row-major V tile.
// The same order is used for the rank index of the low-rank state and for
// tokens in the state contraction.
#include "rola_device.h"

namespace rola {

// ---------------------------------------------------------------- k_setup
// bf16 transposed projections [32][D]; rows >= rank are zero.
__global__ void k_setup(const float *__restrict__ wq, const float *__restrict__ wk, int D, int rank,
                        uint16_t *__restrict__ wqT, uint16_t *__restrict__ wkT) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
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
}

// ---------------------------------------------------------------- fp8 path

// K tile image of one 64-token block (bytes; 64*D per block), [64 keys][D]:
// dim d of a key sits at position
//   p = 64*(d/64) + 32*((d%16)/8) + 8*((d%64)/16) + d%8,
// so that each MFMA lane half reads the 32 dims its Q operand holds (the
// bf16 Q registers, 16 dims per 16-dim step, 8 per lane half) as two
// contiguous 16-byte chunks; chunk c of key row r is stored at
// c ^ ((r / (256/D)) & (D/16 - 1)), conflict-free for 16-lane reads.
// The V codes go to their own [BH][n_pad][D] array as fp16 values, the
// layout of the bf16 path's fp16 copy of V.
template <int D>
static __device__ __forceinline__ int img_k_off(int r, int d) {
  const int rem = d & 63;
  const int p = (d & ~63) + 32 * ((rem & 15) >> 3) + 8 * (rem >> 4) + (rem & 7);
  const int f = (r / (256 / D)) & (D / 16 - 1);
  return r * D + ((((p >> 4) ^ f)) << 4) + (p & 15);
}
// Eight e4m3 codes (the bytes of w, low byte first) as eight fp16 values:
// every e4m3 value is an fp16 value, so the conversion is exact.
static __device__ __forceinline__ u32x4 e4m3x8_f16(uint2 w) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a[0], a[1])),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(b[0], b[1])),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(c[0], c[1])),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(d[0], d[1]))};
}

// ---------------------------------------------------------------- k_pass1
// Grid (nchunks, B*H), 256 threads: each workgroup streams `cpc` consecutive
// 64-token blocks of one (batch, head).  The four waves work independently
// (no barriers):
//   POOL : wave 0 pools Q, wave 1 pools K, straight from global memory.  A
//          lane holds 8 dims (one 16-byte load) of tokens 4r + lane/16
//          (r = 0..15 at D = 128), so the fixed fp32 tree -- pairs at token
//          distance 32, 16, 8, 4 inside the lane, then 2 and 1 across
//          lanes -- runs in place.
//   STATE: waves 2 and 3 take tokens 0-31 and 32-63 of each block: K rows
//          as MFMA operands straight from global memory (one block ahead in
//          registers), b = phi(Wk^T R(k)) on MFMA, then S^T += V^T b and
//          z += b with V^T read transposed from LDS.  Each state wave copies
//          its own 32-token half of V into its own 3-slot LDS ring (two
//          blocks ahead), so it only waits for its own copies.  Per-wave
//          partial sums go to the workspace for a fixed-order reduction.
//   QUANT: (fp8 mode, with POOL) the pooling waves also take the block
//          absmax of Q (its scales) and of K (scales and the block's e4m3 K
//          tile image), and wave 0 then reads the block of V the same way
//          and writes its scales and its codes as fp16 values (see k_quant8
//          for the image layout and rounding).
//   VH:    (bf16 output) the two pooling waves also read V, 32 tokens of
//          each block each, and write its fp16 copy for the attention
//          kernel's PV product, with a range flag per wave (some valid
//          |v| >= 2^16, beyond fp16, or inf).  bf16 values below 2^16 are
//          fp16 values (8 significant bits within 11), so the copy is exact
//          there, down to fp16's subnormal range.  Without POOL: the copy
//          alone.
// Rows past N are read as zero (pooling) or taken from row N-1 (finite
// values; their b is masked to 0).
// bytes of one per-block low-rank state (complement scope): bf16 S^T [D][32]
// (rank in natural order), then fp32 z [32]
static __host__ __device__ constexpr int blk_state_bytes(int D) { return D * 64 + 128; }

template <int D, bool POOL, bool STATE, bool QUANT, bool BLK, bool VH = false>
__global__ __launch_bounds__(256, 2) void k_pass1(Pass1Args args) {
  constexpr int CH = D / 8;       // 16-byte chunks per token row
  constexpr int NS = D / 16;      // MFMA k-steps over head_dim
  constexpr int DT = D / 32;      // d-tiles of the state
  constexpr int VT = 32 * D;      // bf16 elements of a 32-token V half tile
  constexpr int NSTAGE = 3;
  constexpr int VOPS = (32 * CH) / 64;  // DMA ops per lane per half tile
  __shared__ __attribute__((aligned(1024))) uint16_t vring[STATE ? 2 * NSTAGE * VT : 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int bh = blockIdx.y;
  const int b = bh / args.heads, h = bh % args.heads;
  const int64_t base = (int64_t)b * args.stride_b + (int64_t)h * args.stride_h;
  const int c0 = blockIdx.x * args.cpc;
  const int c1 = min(args.nb, c0 + args.cpc);
  const int nblk = c1 - c0;
  const RopeArgsDev ra = args.rope;
  // projection rows and rotary frequencies of the state waves, shared
  __shared__ __attribute__((aligned(16))) uint16_t swk[STATE ? 32 * D : 8];
  __shared__ float sfreq[STATE ? D / 2 : 1];
  if (STATE) {
    for (int e = tid; e < 32 * D / 8; e += 256) ((u32x4 *)swk)[e] = ((const u32x4 *)args.wkT)[e];
    for (int p2 = tid; p2 < D / 2; p2 += 256) sfreq[p2] = rope_freq(2 * p2, ra);
    __syncthreads();  // the only barrier: before the waves take their roles
  }

  // lane layout of the pooling / quantising waves: LPR lanes per token row
  // (8 dims each), TG token groups per load, R loads per block
  constexpr int LPR = D / 8, TG = 64 / LPR, R = 64 / TG;
  const int dl = lane % LPR, tg = lane / LPR;
  // block absmax over this wave's lanes, scale fl32(absmax/448) and inverse
  // fl32(448/absmax) (1 and 1 for an all-zero block)
  auto wave_absmax = [&](float m) __attribute__((always_inline)) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    return m;
  };
  auto e4m3x8 = [&](u32x4 x, float inv) __attribute__((always_inline)) -> uint2 {
    const int w0 = cvt_fp8x2<true>(bflo(x[1]) * inv, bfhi(x[1]) * inv,
                                   cvt_fp8x2<false>(bflo(x[0]) * inv, bfhi(x[0]) * inv, 0));
    const int w1 = cvt_fp8x2<true>(bflo(x[3]) * inv, bfhi(x[3]) * inv,
                                   cvt_fp8x2<false>(bflo(x[2]) * inv, bfhi(x[2]) * inv, 0));
    return make_uint2((uint32_t)w0, (uint32_t)w1);
  };

  // fp8 codes of V block c (wave 0 in fp8 mode, after the block's Q): the
  // block's scale, then its rows of codes as fp16 values (rows past N zero)
  auto quant_v = [&](int c) __attribute__((always_inline)) {
    const uint16_t *X = args.v + base;
    uint16_t *Y = args.vh + (int64_t)bh * args.nb * 64 * D;
    const int valid = min(64, (int)(args.n_tokens - (int64_t)c * 64));
    u32x4 raw[R];
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = TG * r + tg;
      raw[r] = t < valid ? *(const u32x4 *)(X + ((int64_t)c * 64 + t) * args.stride_n + 8 * dl)
                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bflo(raw[r][e])), fabsf(bfhi(raw[r][e]))));
    }
    m = wave_absmax(m);
    const int64_t sidx = (int64_t)bh * args.nb + c;
    const float inv = m > 0.0f ? __fdiv_rn(448.0f, m) : 1.0f;
    if (lane == 0) args.vsc[sidx] = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = TG * r + tg;
      *(u32x4 *)(Y + ((int64_t)c * 64 + t) * D + 8 * dl) = e4m3x8_f16(e4m3x8(raw[r], inv));
    }
  };

  if (wave < 2) {
    if (!POOL && !VH) return;
    // ---- pooling (wave 0: Q, wave 1: K) and, with VH, the fp16 copy of
    // this wave's 32 tokens of each V block (wave 0 tokens 0-31, wave 1
    // tokens 32-63), loaded with the block's Q/K rows
    const uint16_t *X = (wave == 0 ? args.q : args.k) + base;
    const uint16_t *XV = args.v + base;
    uint16_t *YV = VH ? args.vh + (int64_t)bh * args.nb * 64 * D : nullptr;
    float *dst = wave == 0 ? args.qp : args.kp;
    float vmax = 0.0f;  // largest |v| copied (VH)
    for (int i = 0; i < nblk; ++i) {
      const int c = c0 + i;
      const int valid = min(64, (int)(args.n_tokens - (int64_t)c * 64));
      u32x4 vraw[VH ? R / 2 : 1];
      if constexpr (VH) {
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
          const int t = 32 * wave + TG * r + tg;
          vraw[r] = t < valid ? *(const u32x4 *)(XV + ((int64_t)c * 64 + t) * args.stride_n + 8 * dl)
                              : u32x4{0u, 0u, 0u, 0u};
        }
      }
      if constexpr (POOL) {
        auto ld = [&](int t) __attribute__((always_inline)) -> u32x4 {
          return t < valid ? *(const u32x4 *)(X + ((int64_t)c * 64 + t) * args.stride_n + 8 * dl)
                           : u32x4{0u, 0u, 0u, 0u};
        };
        // token distance 32 as the pairs arrive (registers r and r + R/2)
        float x[R / 2][8];
        u32x4 keep[QUANT ? R : 1];  // raw K values for the codes (fp8 mode)
        float amax = 0.0f;
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
          const u32x4 lo = ld(TG * r + tg), hi = ld(TG * (r + R / 2) + tg);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[r][2 * e] = bflo(lo[e]) + bflo(hi[e]);
            x[r][2 * e + 1] = bfhi(lo[e]) + bfhi(hi[e]);
            if (QUANT)
              amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bflo(lo[e])), fabsf(bfhi(lo[e]))),
                                       fmaxf(fabsf(bflo(hi[e])), fabsf(bfhi(hi[e])))));
          }
          if constexpr (QUANT) {
            keep[r] = lo;
            keep[r + R / 2] = hi;
          }
        }
        if constexpr (QUANT) {
          amax = wave_absmax(amax);
          const int64_t sidx = (int64_t)bh * args.nb + c;
          const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
          const float inv = amax > 0.0f ? __fdiv_rn(448.0f, amax) : 1.0f;
          if (wave == 0) {
            if (lane == 0) {
              args.qsc[2 * sidx] = sc;
              args.qsc[2 * sidx + 1] = inv;
            }
          } else {
            if (lane == 0) args.ksc[sidx] = sc;
            uint8_t *kimg = args.kv8 + sidx * (64 * D);
#pragma unroll
            for (int r = 0; r < R; ++r)
              *(uint2 *)(kimg + img_k_off<D>(TG * r + tg, 8 * dl)) = e4m3x8(keep[r], inv);
          }
        }
        // token distances 16 .. TG inside the lane (register r + dist/TG)
#pragma unroll
        for (int dist = 16; dist >= TG; dist >>= 1) {
#pragma unroll
          for (int r = 0; r < dist / TG; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[r][e] = x[r][e] + x[r + dist / TG][e];
        }
        // distances TG/2 .. 1 across lanes (token group tg + dist = lane + dist*LPR)
#pragma unroll
        for (int dist = TG / 2; dist >= 1; dist >>= 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float o = __shfl_xor(x[0][e], dist * LPR, 64);
            x[0][e] = x[0][e] + o;  // meaningful in token group 0 (lanes < LPR)
          }
        }
        if (lane < LPR) {
          const float inv = valid == 64 ? 0.015625f : args.inv_tail;
          float *o = dst + ((int64_t)bh * args.nb + c) * D + 8 * dl;
          *(f32x4 *)o = f32x4{x[0][0] * inv, x[0][1] * inv, x[0][2] * inv, x[0][3] * inv};
          *(f32x4 *)(o + 4) = f32x4{x[0][4] * inv, x[0][5] * inv, x[0][6] * inv, x[0][7] * inv};
        }
      }
      if constexpr (VH) {
#pragma unroll
        for (int r = 0; r < R / 2; ++r) {
          const int t = 32 * wave + TG * r + tg;
          u32x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lo = bflo(vraw[r][e]), hi = bfhi(vraw[r][e]);
            vmax = fmaxf(vmax, fmaxf(fabsf(lo), fabsf(hi)));
            hv[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
          }
          if (t < valid) *(u32x4 *)(YV + ((int64_t)c * 64 + t) * D + 8 * dl) = hv;
        }
      }
      if (QUANT && wave == 0) quant_v(c);
    }
    // the range flag of this wave's half of the chunk
    if constexpr (VH) {
      const bool ovf = __builtin_amdgcn_ballot_w64(!(vmax < 65536.0f)) != 0;
      if (lane == 0) args.vovf[((int64_t)bh * gridDim.x + blockIdx.x) * 2 + wave] = ovf ? 1 : 0;
    }
    return;
  }
  if (!STATE) return;

  // ---- low-rank state.  Default: wave 2 takes tokens 0-31 and wave 3
  // tokens 32-63 of every block and both write chunk partial sums.  BLK
  // (complement scope): wave 2 takes the even and wave 3 the odd blocks of
  // the chunk, each block as two 32-token half tiles in turn, so that one
  // wave holds a whole block's state; it writes every block's state and no
  // chunk partials (the reduction then sums the block states).
  const int tt = wave - 2;
  const uint16_t *Kb = args.k + base, *Vb = args.v + base;
  uint16_t *myring = vring + tt * NSTAGE * VT;
  f32x16 sacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) sacc[i] = f32x16{};
  float zacc = 0.0f;
  // half tile u of this wave: block index (in the chunk) and token half
  const int nu = BLK ? 2 * max(0, (nblk - tt + 1) / 2) : nblk;
  auto blk_of = [&](int u) __attribute__((always_inline)) { return BLK ? tt + 2 * (u >> 1) : u; };
  auto half_of = [&](int u) __attribute__((always_inline)) { return BLK ? (u & 1) : tt; };
  // V half tile u -> slot u % NSTAGE (row-major, chunk-swizzled)
  auto issue_v = [&](int u) __attribute__((always_inline)) {
    const int64_t c = c0 + blk_of(u);
    uint16_t *slot = myring + (u % NSTAGE) * VT;
#pragma unroll
    for (int o = 0; o < VOPS; ++o) {
      const int cidx = o * 64 + lane;
      const int row = cidx / CH, pc = cidx % CH;
      const int64_t src = min(c * 64 + 32 * half_of(u) + row, args.n_tokens - 1) * args.stride_n;
      lds_dma16(Vb + src + ((pc ^ swz_v<D>(row)) * 8), slot + o * 512);
    }
  };
  // K operand rows of half tile u: token 32*half + lane%32, dims 16s + 8g .. +8
  auto load_k = [&](int u, bf16x8 (&kr)[NS]) __attribute__((always_inline)) {
    const int64_t row =
        min((int64_t)(c0 + blk_of(u)) * 64 + 32 * half_of(u) + (lane & 31), args.n_tokens - 1);
    const uint16_t *kp = Kb + row * args.stride_n + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s) kr[s] = *(const bf16x8 *)(kp + 16 * s);
  };
  bf16x8 kcur[NS], knext[NS];
  if (nu > 0) issue_v(0);
  if (nu > 1) issue_v(1);
  if (nu > 0) load_k(0, kcur);
  for (int u = 0; u < nu; ++u) {
    if (u + 2 < nu) issue_v(u + 2);
    if (u + 1 < nu) load_k(u + 1, knext);
    // half tile u: V(u) and K(u) were issued before V(u+2) and K(u+1); vmcnt
    // completes in order, so allow exactly the ops issued after K(u)
    if (u + 2 < nu) wait_vmcnt<VOPS + NS>();
    else if (u + 1 < nu) wait_vmcnt<NS>();
    else wait_vmcnt<0>();
    const int c = c0 + blk_of(u);
    const int hf = half_of(u);
    const int valid = min(64, (int)(args.n_tokens - (int64_t)c * 64));
    const uint16_t *sV = myring + (u % NSTAGE) * VT;
    if constexpr (BLK) {
      if (hf == 0) {  // a new block: its own sums
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) sacc[dt] = f32x16{};
        zacc = 0.0f;
      }
    }
    f32x16 bacc = f32x16{};
    int pt, ph, pw;  // padded rows take the last valid position (their b is masked)
    token_pos(min((int64_t)c * 64 + 32 * hf + (lane & 31), args.n_tokens - 1), ra, pt, ph, pw);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 fr = *(const f32x4 *)&sfreq[8 * s + 4 * g];  // pairs of dims 16s + 8g .. +8
      const float freq4[4] = {fr[0], fr[1], fr[2], fr[3]};
      const bf16x8 kx = rope8(kcur[s], 16 * s + 8 * g, pt, ph, pw, freq4, ra);
      bacc = mfma_bf16(kx, *(const bf16x8 *)&swk[(lane & 31) * D + 16 * s + 8 * g], bacc);
    }
    // phi, mask invalid tokens and rank padding, z, pack as B operand
    const bool rok = (lane & 31) < args.rank;
    bf16x8 bop[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tok = 32 * hf + 8 * (e >> 2) + 4 * g + (e & 3);
      float f = phi(bacc[e]);
      f = (rok && tok < valid) ? f : 0.0f;
      zacc += f;
      bop[e >> 3][e & 7] = (__bf16)f;
    }
    // S^T[d][r] += sum_tok V^T[d][tok] * b[tok][r] over these 32 tokens
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 va = vt_operand<D>(sV, s2, dt, lane);
        sacc[dt] = mfma_bf16(va, bop[s2], sacc[dt]);
      }
    }
    if constexpr (BLK) {
      if (hf == 1) {  // the whole block's state: bf16 S^T [D][32], then fp32 z [32]
        uint8_t *bb = args.blk_state + ((int64_t)bh * args.nb + c) * blk_state_bytes(D);
        uint16_t *bs = (uint16_t *)bb;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int d = 32 * dt + 8 * (e >> 2) + 4 * g + (e & 3);
            bs[d * 32 + (lane & 31)] = __builtin_bit_cast(uint16_t, (__bf16)sacc[dt][e]);
          }
        }
        const float zb = zacc + shfl_xor32(zacc);
        if (lane < 32) ((float *)(bb + D * 64))[lane] = zb;
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) kcur[s] = knext[s];
  }

  if (BLK) return;
  float *part = args.state_part + (((int64_t)bh * gridDim.x + blockIdx.x) * 2 + tt) * (D * 32 + 32);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = 32 * dt + 8 * (e >> 2) + 4 * g + (e & 3);
      part[d * 32 + (lane & 31)] = sacc[dt][e];
    }
  }
  const float zt = zacc + shfl_xor32(zacc);
  if (lane < 32) part[D * 32 + lane] = zt;
}
// ------------------------------------------------------------ k_state_reduce
// Fixed-order sum over the np fp32 partials of each head (chunk-major, then
// token half; or the block-range partials of k_blk_partial), one thread per
// state element.
// Writes St (bf16 [D][32], rank index permuted per 16-group, the A operand
// layout of the apply step), z (fp32 [32]) and, if s32 is set, S^T in fp32
// ([D][32], natural rank order).  Rank columns >= rank are 0.
__global__ __launch_bounds__(256) void k_state_reduce(const float *__restrict__ part, int np,
                                                      int D, int rank, uint16_t *__restrict__ st,
                                                      float *__restrict__ z, float *__restrict__ s32) {
  const int bh = blockIdx.y;
  const int stride = D * 32 + 32;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= stride) return;
  const float *p = part + (int64_t)bh * np * stride + idx;
  // fixed order: eight interleaved partial sums (partial i takes partials
  // i, i+8, ...), then combined pairwise; independent loads keep the
  // memory pipeline full
  float acc8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc8[i] = 0.0f;
  int c = 0;
  for (; c + 8 <= np; c += 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc8[i] += p[(int64_t)(c + i) * stride];
  }
  for (int i = 0; c + i < np; ++i) acc8[i] += p[(int64_t)(c + i) * stride];
  const float acc = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
  if (idx < D * 32) {
    const int d = idx / 32, r = idx % 32;
    const int w = r & 15;
    const int pos = (r & ~15) | ((w < 4) ? w : (w < 8) ? w + 4 : (w < 12) ? w - 4 : w);
    const __bf16 v = (__bf16)(r < rank ? acc : 0.0f);
    st[(int64_t)bh * D * 32 + d * 32 + pos] = __builtin_bit_cast(uint16_t, v);
    if (s32) s32[(int64_t)bh * D * 32 + idx] = r < rank ? acc : 0.0f;
  } else {
    const int r = idx - D * 32;
    z[(int64_t)bh * 32 + r] = r < rank ? acc : 0.0f;
  }
}

// ------------------------------------------------------------ k_blk_partial
// Complement scope, first level of the global state: workgroup (p, bh) sums
// the per-block states (bf16 S^T, fp32 z) of blocks [p*per, (p+1)*per) in
// block order, in fp32, 16 bytes per thread and load, and writes an fp32
// partial in the layout k_state_reduce sums ([D*32] S^T, then [32] z).  The
// global state is thereby the sum of exactly the values the complement
// subtracts.
template <int D>
__global__ __launch_bounds__(256) void k_blk_partial(const uint8_t *__restrict__ blk, int nb, int per,
                                                     float *__restrict__ part) {
  constexpr int BB = D * 64 + 128, SC = D * 4, TC = SC + 8, NK = (TC + 255) / 256;
  const int tid = threadIdx.x, p = blockIdx.x, bh = blockIdx.y;
  const int j0 = p * per, j1 = min(nb, j0 + per);
  const uint8_t *base = blk + (int64_t)bh * nb * BB;
  f32x4 acc[NK][2];
#pragma unroll
  for (int k = 0; k < NK; ++k) acc[k][0] = acc[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = j0; j < j1; ++j) {
    const u32x4 *src = (const u32x4 *)(base + (int64_t)j * BB);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = k * 256 + tid;
      if (c < SC) {
        const u32x4 w = src[c];
        acc[k][0] += f32x4{bflo(w[0]), bfhi(w[0]), bflo(w[1]), bfhi(w[1])};
        acc[k][1] += f32x4{bflo(w[2]), bfhi(w[2]), bflo(w[3]), bfhi(w[3])};
      } else if (c < TC) {
        acc[k][0] += __builtin_bit_cast(f32x4, src[c]);
      }
    }
  }
  float *out = part + ((int64_t)bh * gridDim.x + p) * (D * 32 + 32);
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int c = k * 256 + tid;
    if (c < SC) {
      *(f32x4 *)(out + 8 * c) = acc[k][0];
      *(f32x4 *)(out + 8 * c + 4) = acc[k][1];
    } else if (c < TC) {
      *(f32x4 *)(out + D * 32 + 4 * (c - SC)) = acc[k][0];
    }
  }
}

// ------------------------------------------------------------ k_complement
// Complement scope.  One workgroup per group of query blocks, in the same
// group order and XCD mapping as the attention kernel: it walks the group's
// union list once, adding each listed key block's state (bf16 S^T, fp32 z)
// in fp32 into the sums of the members that kept it (a block shared by
// several members is read once), then writes per member query block
// St_c = S - sum (bf16, the rank-permuted A-operand layout of St) and
// z_c = z - sum.  S and z are the sums of the same block states, so the
// difference is the sum over the unkept blocks up to fp32 rounding.  A query
// block that keeps every block gets zeros: nothing is left for its low-rank
// term.
template <int D, int G>
__global__ __launch_bounds__(256) void k_complement(CompArgs a) {
  constexpr int BB = D * 64 + 128;      // bytes per block state
  constexpr int SC = D * 4;             // 16-byte chunks of S^T (8 bf16 each)
  constexpr int TC = SC + 8;            // plus the z chunks (4 floats each)
  constexpr int NK = (TC + 255) / 256;  // chunks per thread
  constexpr int UN = 4;                 // list entries loaded together
  const int tid = threadIdx.x;
  const int64_t L = blockIdx.x;
  const int64_t sidx = L / 8;
  const int64_t bh64 = sidx / a.groups_per_xcd;
  const int64_t group = (L % 8) * a.groups_per_xcd + sidx % a.groups_per_xcd;
  if (bh64 >= a.bh_count || group >= a.ngroups) return;
  const int bh = (int)bh64;
  const int64_t gidx = (int64_t)bh * a.ngroups + group;
  const int32_t *list = a.ulist + gidx * a.list_stride;
  const int U = a.ucount[gidx];
  const uint8_t *blk = a.blk + (int64_t)bh * a.nb * BB;
  // per member and chunk: ranks r0..r0+3 and r0+4..r0+7 of an S^T row, or
  // (the z chunk) four z values and zeros
  f32x4 acc[G][NK][2];
#pragma unroll
  for (int m = 0; m < G; ++m)
#pragma unroll
    for (int k = 0; k < NK; ++k) acc[m][k][0] = acc[m][k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int u0 = 0; u0 < U; u0 += UN) {
    u32x4 x[UN][NK];
    int msk[UN];
#pragma unroll
    for (int i = 0; i < UN; ++i) {
      const bool in = u0 + i < U;
      const int e = in ? list[u0 + i] : 0;
      msk[i] = in ? (e >> 16) : 0;  // entries past the list add nothing
      const u32x4 *src = (const u32x4 *)(blk + (int64_t)(e & 0xffff) * BB);
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int c = k * 256 + tid;
        x[i][k] = c < TC ? src[c] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < UN; ++i) {
      f32x4 f[NK][2];
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const u32x4 w = x[i][k];
        if (k * 256 + tid < SC) {
          f[k][0] = f32x4{bflo(w[0]), bfhi(w[0]), bflo(w[1]), bfhi(w[1])};
          f[k][1] = f32x4{bflo(w[2]), bfhi(w[2]), bflo(w[3]), bfhi(w[3])};
        } else {
          f[k][0] = __builtin_bit_cast(f32x4, w);
          f[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int m = 0; m < G; ++m)
        if ((msk[i] >> m) & 1)
#pragma unroll
          for (int k = 0; k < NK; ++k) {
            acc[m][k][0] += f[k][0];
            acc[m][k][1] += f[k][1];
          }
    }
  }
  const float *sg = a.s32 + (int64_t)bh * D * 32;
  const float *zg = a.z + (int64_t)bh * 32;
  const bool empty = a.kb >= a.nb;
#pragma unroll
  for (int m = 0; m < G; ++m) {
    const int qb = a.ugroup[gidx * G + m];
    if (qb < 0) continue;
    const int64_t qi = (int64_t)bh * a.nb + qb;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = k * 256 + tid;
      if (c < SC) {
        // S^T row d, ranks r0 .. r0+7 -> two 8-byte groups of the permuted St
        const int d = c >> 2, r0 = 8 * (c & 3);
        const f32x4 g0 = *(const f32x4 *)(sg + d * 32 + r0);
        const f32x4 g1 = *(const f32x4 *)(sg + d * 32 + r0 + 4);
        const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 d0 = empty ? zero : g0 - acc[m][k][0], d1 = empty ? zero : g1 - acc[m][k][1];
        const float v[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        uint2 o[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const __bf16 b0 = (__bf16)v[4 * h], b1 = (__bf16)v[4 * h + 1], b2 = (__bf16)v[4 * h + 2],
                       b3 = (__bf16)v[4 * h + 3];
          o[h].x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
          o[h].y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        }
        // ranks 4-7 and 8-11 of each 16-group trade places
        const int pa = (r0 & 8) ? r0 - 4 : r0, pb = (r0 & 8) ? r0 + 4 : r0 + 8;
        uint16_t *so = a.stc + qi * D * 32 + d * 32;
        *(uint2 *)(so + pa) = o[0];
        *(uint2 *)(so + pb) = o[1];
        if (a.sdc) {
          // the backward's [32][D] operand of S dnum: d at its permuted
          // position (the permutation is its own inverse), hi + lo
          const int pd = perm16_key_of_pos(d);
          uint16_t *hi = a.sdc + qi * 32 * D + pd, *lo = hi + a.bh_count * a.nb * 32LL * D;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 hv = (__bf16)v[e];
            hi[(r0 + e) * D] = __builtin_bit_cast(uint16_t, hv);
            lo[(r0 + e) * D] = __builtin_bit_cast(uint16_t, (__bf16)(v[e] - (float)hv));
          }
        }
      } else if (c < TC) {
        const int r = 4 * (c - SC);
        const f32x4 zz = *(const f32x4 *)(zg + r);
        *(f32x4 *)(a.zc + qi * 32 + r) = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : zz - acc[m][k][0];
      }
    }
  }
}

// --------------------------------------------------------------- k_scores
// s[bh][i][j] = sequential fma chain over d of Qp[i][d] * Kp[j][d] from +0.0.
// One workgroup per 64x64 tile of (i, j); thread t computes rows
// 4*(t/16)..+3 by keys 4*(t%16)..+3.  Qp and Kp are staged through LDS in
// 16-dim chunks, transposed ([d][block]), so each d step is two 16-byte LDS
// reads and 16 FMAs.  Chunks are taken in increasing d, so every element's
// chain keeps the order d = 0..D-1.
template <int D>
__global__ __launch_bounds__(256) void k_scores(const float *__restrict__ qp,
                                                const float *__restrict__ kp, float *__restrict__ s,
                                                int nb) {
#pragma clang fp contract(off)
  __shared__ f32x4 qs[16][16];  // [d in chunk][row group]: 4 rows per float4
  __shared__ f32x4 ks[16][16];  // [d in chunk][key group]
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  const int tr = tid >> 4, tc = tid & 15;
  const float *qb = qp + (int64_t)bh * nb * D;
  const float *kb = kp + (int64_t)bh * nb * D;
  // staging: thread t copies 4 dims (d4 = t%4) of block row t/4
  const int srow = tid >> 2, sd4 = tid & 3;
  const int qrow = min(i0 + srow, nb - 1), krow = min(j0 + srow, nb - 1);
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;
  // the chunk being staged is loaded one chunk ahead (its latency under the
  // FMAs of the previous chunk)
  f32x4 qv = *(const f32x4 *)(qb + (int64_t)qrow * D + 4 * sd4);
  f32x4 kv = *(const f32x4 *)(kb + (int64_t)krow * D + 4 * sd4);
  for (int dc = 0; dc < D; dc += 16) {
    __syncthreads();  // previous chunk fully read
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ((float *)&qs[4 * sd4 + e][srow >> 2])[srow & 3] = qv[e];
      ((float *)&ks[4 * sd4 + e][srow >> 2])[srow & 3] = kv[e];
    }
    if (dc + 16 < D) {
      qv = *(const f32x4 *)(qb + (int64_t)qrow * D + dc + 16 + 4 * sd4);
      kv = *(const f32x4 *)(kb + (int64_t)krow * D + dc + 16 + 4 * sd4);
    }
    __syncthreads();
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const f32x4 a = qs[d][tr], b = ks[d][tc];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(a[r], b[c], acc[r][c]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * tr + r;
    if (i >= nb) break;
    float *row = s + ((int64_t)bh * nb + i) * nb;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + 4 * tc + c;
      if (j < nb) row[j] = acc[r][c];
    }
  }
}

// ----------------------------------------------------------------- k_topk
// One wave per score row: order-preserving uint32 keys (-0.0 folded into
// +0.0), the kb-th largest key T, then emit, in ascending index order, every
// j with key > T and the lowest-index ties key == T.
//  - T comes from a bitwise search (from the top bit down, keep a bit when at
//    least kb keys reach the prefix with it set).
//  - For kb <= 64 the search first narrows the row: the kb-th largest of the
//    64 lane maxima, T_sub, is at most T (those maxima are a subset of the
//    row), so every key >= T is a key >= T_sub.  When at most 128 keys reach
//    T_sub they are compacted into two per lane through LDS and the search
//    runs over them alone; otherwise over the whole row.
static __device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// the kb-th largest of the wave's keys k[0..N) (all lanes), by bitwise search
template <int N>
static __device__ __forceinline__ uint32_t kth_largest(const uint32_t *k, int kb) {
  uint32_t prefix = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < N; ++m) cnt += __popcll(__ballot(k[m] >= cand));
    if (cnt >= kb) prefix = cand;
  }
  return prefix;
}

template <int PER>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ s, int32_t *__restrict__ map,
                                              int nb, int kb, int64_t rows) {
  __shared__ uint32_t cand[4][128];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  if (row >= rows) return;
  const float *sr = s + row * nb;
  uint32_t key[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int j = m * 64 + lane;
    key[m] = j < nb ? order_key(sr[j]) : 0u;  // real keys are >= 0x007fffff
  }
  uint32_t T;
  bool narrowed = false;
  if (kb <= 64) {
    uint32_t mx = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) mx = max(mx, key[m]);
    const uint32_t tsub = kth_largest<1>(&mx, kb);
    int total = 0;
#pragma unroll
    for (int m = 0; m < PER; ++m) total += __popcll(__ballot(key[m] >= tsub));
    if (total <= 128) {
      int base = 0;
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const bool c = key[m] >= tsub;
        const uint64_t cm = __ballot(c);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(cm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cm, 0u));
        if (c) cand[w][base + (int)below] = key[m];
        base += __popcll(cm);
      }
      __builtin_amdgcn_wave_barrier();
      uint32_t ck[2];
      ck[0] = lane < total ? cand[w][lane] : 0u;
      ck[1] = 64 + lane < total ? cand[w][64 + lane] : 0u;
      T = kth_largest<2>(ck, kb);
      narrowed = true;
    }
  }
  if (!narrowed) T = kth_largest<PER>(key, kb);
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

// ---------------------------------------------------------------- k_order
// Orders each (batch, head)'s query blocks by the first two entries of their
// (ascending) block maps, so that query blocks keeping similar key blocks
// become neighbours, and writes the groups of G members.  Without a map
// (kb == 0, low-rank only) the order is the identity.  Rank sort: the
// position of block i is #{j : (key_j, j) < (key_i, i)}.  Grid (ceil(nb /
// kOrderPer), batch*heads); eight lanes share one block i, each counting a
// strided eighth of the j, and combine their counts with shuffles.
constexpr int kOrderPer = 128;
__global__ __launch_bounds__(1024) void k_order(const int32_t *__restrict__ map, int nb, int kb, int G,
                                                int ngroups, int32_t *__restrict__ ugroup) {
  extern __shared__ uint32_t key[];  // [nb]
  const int bh = blockIdx.y;
  const int32_t *mb = kb > 0 ? map + (int64_t)bh * nb * kb : nullptr;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) {
    uint32_t key_i = (uint32_t)i;
    if (kb > 0) {
      const uint32_t a = (uint32_t)min(max(mb[(int64_t)i * kb], 0), nb - 1);
      const uint32_t b = kb > 1 ? (uint32_t)min(max(mb[(int64_t)i * kb + 1], 0), nb - 1) : 0u;
      key_i = (a << 12) | b;
    }
    key[i] = key_i;
  }
  __syncthreads();
  int32_t *ug = ugroup + (int64_t)bh * ngroups * G;
  const int i = blockIdx.x * kOrderPer + (int)(threadIdx.x >> 3), part = (int)(threadIdx.x & 7);
  const uint32_t ki = i < nb ? key[i] : 0u;
  int rank = 0;
  if (i < nb) {
    for (int j = part; j < nb; j += 8) {
      const uint32_t kj = key[j];
      rank += (kj < ki) || (kj == ki && j < i);
    }
  }
  rank += __shfl_xor(rank, 1, 64);
  rank += __shfl_xor(rank, 2, 64);
  rank += __shfl_xor(rank, 4, 64);
  if (i < nb && part == 0) ug[rank] = i;
  if (blockIdx.x == 0)
    for (int p = nb + threadIdx.x; p < ngroups * G; p += blockDim.x) ug[p] = -1;
}

// ---------------------------------------------------------------- k_group
// Refines the grouping inside windows of kGroupWin consecutive positions of
// the k_order sequence (one wave per window, windows independent): groups
// are formed greedily, seeded by the first unassigned query block in window
// order, each next member being the unassigned block whose map shares the
// most key blocks with the group's union so far (ties to the earlier one).
// Fewer distinct key blocks per group means fewer K/V tiles to stream and
// fewer waves idle on a tile.  Windows are multiples of G, so group
// boundaries stay aligned; padding entries (-1) stay at the end.  Used for
// kb <= kGroupMaxKb (maps cached in LDS as 16-bit ids).
extern "C" __device__ int __ockl_wfred_max_i32(int);

constexpr int kGroupWin = 64;
constexpr int kGroupMaxKb = 64;

// One wave per window, window position c = lane.  Each lane keeps its own
// map (up to kGroupMaxKb key blocks) in registers; the group's union is a
// bitset in LDS.  At every greedy step each live lane recounts its key
// blocks present in the union (all bitset reads independent, so one LDS
// round trip per step), and a max-reduction over the wave picks the next
// member.  The maps are also staged in LDS so that a new member's key blocks
// enter the union in one step (one lane per key block).  KBM >= kb bounds the
// unrolled recount: all KBM reads are issued without branches (entries past
// kb are masked afterwards), so they overlap.  Dynamic LDS: the union bitset.
template <int KBM>
__global__ __launch_bounds__(64) void k_group(const int32_t *__restrict__ map, int nb, int kb, int G,
                                              int ngroups, int32_t *__restrict__ ugroup) {
  extern __shared__ uint32_t inu[];                     // [ceil(nb/32)]
  __shared__ uint16_t cmap[kGroupWin * kGroupMaxKb];    // maps of the window positions
  const int lane = threadIdx.x;
  const int bh = blockIdx.y;
  const int total = ngroups * G;
  const int w0 = blockIdx.x * kGroupWin;
  if (w0 >= total) return;
  const int wn = min(kGroupWin, total - w0);
  int32_t *ug = ugroup + (int64_t)bh * total + w0;
  const int32_t *mb = map + (int64_t)bh * nb * kb;
  const int nwords = (nb + 31) / 32;
  const int qb = lane < wn ? ug[lane] : -1;
  // stage the window's maps: entries e = c*kb + t spread over the lanes,
  // four loads in flight
  const int nent = wn * kb;
  for (int e0 = 0; e0 < nent; e0 += 256) {
    int jv[4], cv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + 64 * u + lane;
      const int c = e < nent ? e / kb : 0;
      const int qc = __shfl(qb, c, 64);
      cv[u] = (e < nent && qc >= 0) ? c : -1;
      jv[u] = cv[u] >= 0 ? mb[(int64_t)qc * kb + (e - c * kb)] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (cv[u] >= 0) cmap[e0 + 64 * u + lane] = (uint16_t)min(max(jv[u], 0), nb - 1);
  }
  __syncthreads();
  // this lane's map in registers, as (word, bit) of the union bitset
  uint32_t kw[KBM];
#pragma unroll
  for (int t = 0; t < KBM; ++t) {
    const int j = (t < kb && qb >= 0) ? (int)cmap[lane * kb + t] : 0;
    kw[t] = ((uint32_t)(j >> 5) << 5) | (uint32_t)(j & 31);
  }
  uint64_t live = __builtin_amdgcn_ballot_w64(qb >= 0);
  // the key blocks of position c join the union (lane t < kb takes entry t)
  auto add_member = [&](int c) {
    if (lane < kb) {
      const int j = cmap[c * kb + lane];
      atomicOr(&inu[j >> 5], 1u << (j & 31));
    }
    __syncthreads();  // the union bits are complete before the next reads
  };
  // key blocks of this lane's map present in the union
  auto score = [&]() -> int {
    uint32_t bits[KBM];
#pragma unroll
    for (int t = 0; t < KBM; ++t) bits[t] = inu[kw[t] >> 5];
    int sc = 0;
#pragma unroll
    for (int t = 0; t < KBM; ++t) sc += (t < kb) ? (int)((bits[t] >> (kw[t] & 31)) & 1u) : 0;
    return sc;
  };
  int32_t outv = -1;  // regrouped sequence: position p held by lane p
  int outp = 0;
  while (live) {
    const int sd = __builtin_ctzll(live);
    for (int w = lane; w < nwords; w += 64) inu[w] = 0u;
    __syncthreads();
    const int vs = __shfl(qb, sd, 64);  // with every lane active
    if (lane == outp) outv = vs;
    live &= ~(1ull << sd);
    add_member(sd);
    for (int members = 1; members < G && live; ++members) {
      // key = score*64 + (63 - position): most shared key blocks, then earliest
      int best = ((live >> lane) & 1ull) ? score() * 64 + (63 - lane) : -1;
      best = __ockl_wfred_max_i32(best);  // wave-wide max on DPP
      const int c = 63 - (best & 63);
      const int v = __shfl(qb, c, 64);
      if (lane == outp + members) outv = v;
      live &= ~(1ull << c);
      if (members + 1 < G) add_member(c);
    }
    outp += G;
    __syncthreads();  // every lane's score reads are done before the union is cleared
  }
  if (lane < wn) ug[lane] = outv;
}

// ---------------------------------------------------------------- k_union
// One wave per group: the members' maps are folded into per-key-block member
// masks in LDS (4 key blocks per word, one byte each), then compacted into
// the group's list of (key block | mask << 16).  The attention kernels take
// the list two tiles per barrier, and their SIMDs host members {0, 2} and
// {1, 3} in pairs, so the list is ordered to give each consecutive pair of
// tiles an even load on the two SIMD pairs: entries are ranked by
// d = |mask & {0,2}| - |mask & {1,3}| (stable in key-block order), and the
// ranked sequence is emitted from both ends alternately (lowest, highest,
// second lowest, second highest, ...).
constexpr int kUnionWaves = 8;

__global__ __launch_bounds__(64 * kUnionWaves) void k_union(const int32_t *__restrict__ map, int nb,
                                                            int kb, int G, int ngroups, int list_stride,
                                                            const int32_t *__restrict__ ugroup,
                                                            int32_t *__restrict__ ucount,
                                                            int32_t *__restrict__ ulist) {
  extern __shared__ uint32_t smask[];  // [kUnionWaves][nbw]
  const int nbw = (nb + 3) / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y;
  const int gi = blockIdx.x * kUnionWaves + wave;
  if (gi >= ngroups) return;  // per wave; no workgroup barrier follows
  uint32_t *mw = smask + wave * nbw;
  for (int w = lane; w < nbw; w += 64) mw[w] = 0u;
  const int64_t gidx = (int64_t)bh * ngroups + gi;
  const int32_t *mb = map + (int64_t)bh * nb * kb;
  for (int e = lane; e < G * kb; e += 64) {
    const int m = e / kb, t = e - m * kb;
    const int qb = ugroup[gidx * G + m];
    if (qb < 0) continue;
    const int j = min(max(mb[(int64_t)qb * kb + t], 0), nb - 1);
    atomicOr(&mw[j >> 2], 1u << ((j & 3) * 8 + m));
  }
  // lane owns words [lane*per, lane*per + per); per-lane counts per rank
  // class d + 2 in 0..4, then exclusive scans across lanes
  auto dclass = [](uint32_t msk) -> int {
    return __builtin_popcount(msk & 5u) - __builtin_popcount(msk & 10u) + 2;
  };
  const int per = (nbw + 63) / 64;
  int cnt[5] = {0, 0, 0, 0, 0};
  for (int w = lane * per; w < min(nbw, lane * per + per); ++w) {
    const uint32_t x = mw[w];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t msk = (x >> (8 * q)) & 0xffu;
      if (msk) {
        const int dc = dclass(msk);
#pragma unroll
        for (int c = 0; c < 5; ++c) cnt[c] += (dc == c);
      }
    }
  }
  int rank[5], base = 0, U = 0;
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    int incl = cnt[c];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int total = __shfl(incl, 63, 64);
    rank[c] = base + incl - cnt[c];  // this lane's first sorted index in class c
    base += total;
  }
  U = base;
  int32_t *out = ulist + gidx * list_stride;
  for (int w = lane * per; w < min(nbw, lane * per + per); ++w) {
    const uint32_t x = mw[w];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t msk = (x >> (8 * q)) & 0xffu;
      if (msk) {
        const int dc = dclass(msk);
        int i = 0;
#pragma unroll
        for (int c = 0; c < 5; ++c)
          if (dc == c) i = rank[c]++;
        const int pos = i < (U + 1) / 2 ? 2 * i : 2 * (U - 1 - i) + 1;
        out[pos] = (4 * w + q) | (int)(msk << 16);
      }
    }
  }
  if (lane == 0) ucount[gidx] = U;
}

// Epilogue shared by the bf16 and fp8 attention kernels: low-rank apply
// O^T += g St a / (a^T z) with a = phi(Wq^T R(q)) (Q in registers as the
// bf16 B operand) and g the optional output gate (1 without one), then the write of query row n (bf16 or fp32, optional
// accumulate; rows >= N written as zero).
template <int D, bool LOWRANK, bool ACCUM, bool OUTF32>
static __device__ __forceinline__ void attn_finish(const AttnArgs &args, const bf16x8 *qreg,
                                                   f32x16 *oacc, int64_t n, int64_t base, int bh,
                                                   int lane, const float *sfreq) {
  constexpr int NS = D / 16;
  constexpr int DT = D / 32;
  const int g = lane >> 5;
  if (LOWRANK) {
    // a^T = Wq^T R(q): A = Wq^T (rows r), B = rotated Q (cols query)
    int pt, ph, pw;  // padded rows take the last valid position (they are written as 0)
    token_pos(n < args.n_tokens ? n : args.n_tokens - 1, args.rope, pt, ph, pw);
    f32x16 aacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 fr = *(const f32x4 *)&sfreq[8 * s + 4 * g];  // pairs of dims 16s + 8g .. +8
      const float freq[4] = {fr[0], fr[1], fr[2], fr[3]};
      const bf16x8 qr = rope8(qreg[s], 16 * s + 8 * g, pt, ph, pw, freq, args.rope);
      const bf16x8 wa = *(const bf16x8 *)(args.wqT + (lane & 31) * D + 16 * s + 8 * g);
      aacc = mfma_bf16(wa, qr, aacc);
    }
    // one state per (batch, head), or per query block in the complement scope
    const int64_t si = args.complement ? (int64_t)bh * args.nb + n / 64 : (int64_t)bh;
    const f32x4 *zb = (const f32x4 *)(args.z + si * 32);
    float den = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 zq = zb[2 * q + g];  // z[8q + 4g .. +4]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * q + j, r = 8 * q + 4 * g + j;
        const float a = r < args.rank ? phi(aacc[i]) : 0.0f;
        aacc[i] = a;
        den += a * zq[j];
      }
    }
    den += shfl_xor32(den);
    float inv_den = den > 0.0f ? 1.0f / den : 0.0f;  // 0: an empty complement
    if (args.gate) {
      // learned output gate sigmoid(q . w + b) of this query on the low-rank
      // term; each half-wave holds half of the query's dims
      float u = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const f32x4 w0 = *(const f32x4 *)(args.gate + 16 * s + 8 * g);
        const f32x4 w1 = *(const f32x4 *)(args.gate + 16 * s + 8 * g + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u += (float)qreg[s][e] * w0[e];
          u += (float)qreg[s][4 + e] * w1[e];
        }
      }
      u += shfl_xor32(u);
      inv_den *= 1.0f / (1.0f + __expf(-(u + args.gate[D])));
    }
    bf16x8 aop[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) aop[i >> 3][i & 7] = (__bf16)(aacc[i] * inv_den);
    const uint16_t *stb = args.st + si * D * 32;
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

// ----------------------------------------------------------------- k_attn
// One workgroup per group of G query blocks of one (batch, head); waves
// 2m and 2m+1 own query rows 0-31 and 32-63 of member m, one query per lane
// column.  The workgroup walks the group's union list; each listed key
// block's K and V tiles (row-major, chunk-swizzled) are copied global->LDS
// directly (16 B per lane) into an S-slot ring,
// S-1 tiles ahead of the one being consumed, and every member that kept
// the block runs S^T = K Q^T, the online softmax and O^T += V^T P^T on it.
// Workgroups are mapped so that all XCDs work on the same head at a time and
// each XCD takes a contiguous run of similar groups (shared L2 lines).
// Two forms of the PV product:
//   EXACT (fp32 output, and the backward's recompute of the sparse branch):
//     V is the caller's bf16 tensor; the row sums add the fp32 weights and
//     each weight enters the PV product as a bf16 pair hi + lo, so that O and
//     the log-sum-exp agree with fp32 weights to about 16 bits.
//   otherwise (bf16 output): V is pass 1's fp16 copy (exact for |v| < 2^16)
//     and each weight is one fp16 value (11 significant bits, against 8 for
//     a bf16 weight, whose rounding alone would cost up to about 2e-2 of the
//     output RMS on these shapes), on the f16 MFMA at the bf16 rate.  Heads
//     whose copy would overflow (a |v| >= 2^16, flagged per pass-1 chunk) are
//     skipped here and computed by the EXACT form launched after it with the
//     same flags, which then runs those heads only.
template <int D, int G, int S, bool SPARSE, bool LOWRANK, bool ACCUM, bool OUTF32, bool EXACT = OUTF32,
          bool FALLBACK = false>
__global__ __launch_bounds__(128 * G, 2) void k_attn(AttnArgs args) {
  static_assert(!FALLBACK || (SPARSE && EXACT), "the fallback is the EXACT form of the sparse branch");
  constexpr int CH = D / 8;
  constexpr int NS = D / 16;  // k-steps over head_dim
  constexpr int DT = D / 32;  // output d-tiles
  constexpr int NT = 128 * G;
  constexpr int TILE = 64 * D;                // bf16 elements per K (or V^T) tile
  constexpr int OPS = (64 * CH) / NT;         // DMA ops per thread per tensor per tile
  static_assert(OPS >= 1 && (64 * CH) % NT == 0, "tile split");
  static_assert(S == 2 || S == 4, "ring depth");
  constexpr int LMAX = 2048;  // union-list entries staged in LDS (longer lists read the tail from HBM)
  __shared__ __attribute__((aligned(1024))) uint16_t ring[SPARSE ? S * 2 * TILE : 8];
  __shared__ int32_t slist[SPARSE ? LMAX + 8 : 4];  // + room for the reads ahead past the end
  __shared__ __attribute__((aligned(16))) float sfreq[D / 2];  // rotary inverse frequency per pair

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int member = wave >> 1, half = wave & 1;
  // any range flag of head bh's fp16 V copy set
  auto v_overflow = [&](int bh) __attribute__((always_inline)) -> bool {
    int f = 0;
    for (int i = lane; i < args.nflags; i += 64) f |= args.vovf[(int64_t)bh * args.nflags + i];
    return __builtin_amdgcn_ballot_w64(f != 0) != 0;
  };
  // one group of query blocks of head bh
  auto run_group = [&](const int bh, const int64_t group) __attribute__((always_inline)) {
  const int64_t gidx = (int64_t)bh * args.ngroups + group;
  // wave-uniform values through the scalar cache (the schedule is written by
  // earlier kernels and only read here)
  typedef const __attribute__((address_space(4))) int32_t *cint_p;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qb = ((cint_p)args.ugroup)[gidx * G + (wave_u >> 1)];
  const bool active = qb >= 0;
  const int b = bh / args.heads, h = bh % args.heads;
  const int64_t base = (int64_t)b * args.stride_b + (int64_t)h * args.stride_h;
  const int64_t n = (int64_t)(active ? qb : 0) * 64 + 32 * half + (lane & 31);

  bf16x8 qreg[NS];
  const uint16_t *qrow = args.q + base + n * args.stride_n;
  if (!SPARSE) {
#pragma unroll
    for (int s = 0; s < NS; ++s) qreg[s] = *(const bf16x8 *)(qrow + 16 * s + 8 * g);
    wait_vmcnt<0>();
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  for (int p2 = tid; p2 < D / 2; p2 += NT) sfreq[p2] = rope_freq(2 * p2, args.rope);
  if (!SPARSE) __syncthreads();  // the sparse path's list staging synchronises

  if (SPARSE) {
    const int32_t *list = args.ulist + gidx * args.list_stride;
    const int U = ((cint_p)args.ucount)[gidx];
    const uint16_t *Kb = args.k + base;
    // V: the caller's bf16 tensor, or its fp16 copy [BH][n_pad][D]
    const uint16_t *Vb = EXACT ? args.v + base : args.vh + (int64_t)bh * args.nb * 64 * D;
    const int64_t vstride = EXACT ? args.stride_n : D;
    const float c = args.scale_log2e;
    // per-lane LDS element offsets of the MFMA operands inside a tile:
    // K rows l%32 (+32 rows for the second key tile) at chunk 2s+g;
    // V^T transposed-read rows 4g + (l%16)/4 (+16 per k-step, +8 for the
    // second half), dims 32dt + 16((l/16)%2) + 4(l%4)
    int koff[NS], voff[DT];
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    uint32_t gk[OPS], gv[OPS];  // this lane's byte offsets inside a key block
#pragma unroll
    for (int o = 0; o < OPS; ++o) {
      const int cidx = o * NT + tid;
      const int row = cidx / CH, pc = cidx % CH;
      gk[o] = (uint32_t)(((int64_t)row * args.stride_n + ((pc ^ swz_k<D>(row)) * 8)) * 2);
      gv[o] = (uint32_t)(((int64_t)row * vstride + ((pc ^ swz_v<D>(row)) * 8)) * 2);
    }
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int row = lane & 31;
      koff[s2] = row * D + (((2 * s2 + g) ^ swz_k<D>(row)) * 8);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int i = lane & 15, dhalf = (lane >> 4) & 1;
      const int dstart = 32 * dt + 16 * dhalf + 4 * (i & 3);
      const int r0 = 4 * g + (i >> 2);
      voff[dt] = r0 * D + (((dstart >> 3) ^ swz_v<D>(r0)) << 3) + (dstart & 7);
    }
    auto issue_j = [&](int t, int j) {
      uint16_t *slot = ring + (t % S) * (2 * TILE);
      const int64_t jrow = (int64_t)j * 64;
      if (jrow + 64 <= args.n_tokens) {
        const uint16_t *kj = Kb + jrow * args.stride_n, *vj = Vb + jrow * vstride;
        const uint32_t m0 = ring_lds + (uint32_t)((t % S) * (2 * TILE) * 2) + (uint32_t)wave_s * 1024u;
#pragma unroll
        for (int o = 0; o < OPS; ++o) {
          lds_dma16_m0(kj, gk[o], m0 + (uint32_t)(o * NT * 16));
          lds_dma16_m0(vj, gv[o], m0 + (uint32_t)(TILE * 2 + o * NT * 16));
        }
      } else {
#pragma unroll
        for (int o = 0; o < OPS; ++o) {
          const int cidx = o * NT + tid;
          const int row = cidx / CH, pc = cidx % CH;
          // rows past N (tail block) are copied from row N-1: finite
          // values, masked out of the softmax
          const int64_t src = min(jrow + row, args.n_tokens - 1);
          lds_dma16(Kb + src * args.stride_n + ((pc ^ swz_k<D>(row)) * 8), slot + (o * NT + wave * 64) * 8);
          lds_dma16(Vb + src * vstride + ((pc ^ swz_v<D>(row)) * 8), slot + TILE + (o * NT + wave * 64) * 8);
        }
      }
    };
    // Prologue, one memory round trip: the copies of tiles 0 and 1 (their
    // key blocks read through the scalar cache), then Q and the list, all in
    // flight together.  The list is staged in LDS: a global load inside the
    // loop would need vmcnt(0), which also drains the prefetched tiles.
    // Lists longer than LMAX (keep ratios near 1) take a second copy of the
    // loop that reads the list from HBM.
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (t < U) issue_j(t, ((cint_p)list)[t] & 0xffff);
#pragma unroll
    for (int s = 0; s < NS; ++s) qreg[s] = *(const bf16x8 *)(qrow + 16 * s + 8 * g);
    {
      int32_t lv[(LMAX + NT - 1) / NT];
#pragma unroll
      for (int r = 0; r < (LMAX + NT - 1) / NT; ++r) {
        const int i = r * NT + tid;
        lv[r] = i < min(U, LMAX) ? list[i] : 0;
      }
      // the fp16 form leaves flagged heads to the bf16 form (checked here,
      // under the prologue's copies, which are complete before the return)
      const bool skip = !EXACT && args.vovf && v_overflow(bh);
      wait_vmcnt<0>();
      if (skip) return;
#pragma unroll
      for (int r = 0; r < (LMAX + NT - 1) / NT; ++r) {
        const int i = r * NT + tid;
        if (i < min(U, LMAX)) slist[i] = lv[r];
      }
    }
    __syncthreads();  // tiles 0 and 1 and the list complete for every wave
    auto main_loop = [&](auto lds_tag) {
      constexpr bool FROM_LDS = decltype(lds_tag)::value;
      auto entry = [&](int t) -> int {
        if constexpr (FROM_LDS) return slist[t];
        else return list[t];
      };
      auto issue = [&](int t) { issue_j(t, __builtin_amdgcn_readfirstlane(entry(t) & 0xffff)); };
      // one listed tile t (list entry ent) for this wave's 32 query rows
      auto tile = [&](int t, int ent) __attribute__((always_inline)) {
        const int j = ent & 0xffff;
        const uint16_t *sK = ring + (t % S) * (2 * TILE);
        const uint16_t *sV = sK + TILE;
        // ---- S^T = K Q^T: two independent 32-key chains
        f32x16 sacc0 = f32x16{}, sacc1 = f32x16{};
        // all K operands of the tile (2*NS 16-byte LDS reads) are issued
        // before the first MFMA (the scheduler would otherwise wait on each
        // read just before its MFMA); the two key halves' chains interleave
        {
          bf16x8 ka[NS], kb2[NS];
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            ka[s] = *(const bf16x8 *)(sK + koff[s]);
            kb2[s] = *(const bf16x8 *)(sK + koff[s] + 32 * D);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            sacc0 = mfma_bf16(ka[s], qreg[s], sacc0);
            sacc1 = mfma_bf16(kb2[s], qreg[s], sacc1);
          }
        }
        // keys >= N masked in the tail block (key 8(i/4) + 4g + i%4 of the
        // accumulator; compared as immediates against a per-lane limit)
        if ((int64_t)(j + 1) * 64 > args.n_tokens) {
          const int lim = (int)(args.n_tokens - (int64_t)j * 64) - 4 * g;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kc = 8 * (i >> 2) + (i & 3);
            if (kc >= lim) sacc0[i] = -INFINITY;
            if (kc + 32 >= lim) sacc1[i] = -INFINITY;
          }
        }
        // ---- online softmax, base 2, against a lazy reference: weights
        // are exp2(s*c - m_ref) with m_ref an integer that moves only when the
        // tile max exceeds it by more than W (or on the first tile), so O is
        // rarely rescaled and the rescale, when it happens, is by an exact
        // power of two.  Weights stay below 2^W: W = 64 for the fp32 weights
        // of the EXACT form, W = 15 for fp16 weights (largest finite 65504).
        // fp16 weights below 2^-24 vanish; relative to the row sum (at least
        // 1/2) they are negligible.
        constexpr float W = EXACT ? 64.0f : 15.0f;
        float mx0 = -INFINITY, mx1 = -INFINITY, mx2 = -INFINITY, mx3 = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          mx0 = fmaxf(mx0, sacc0[i]);
          mx1 = fmaxf(mx1, sacc1[i]);
          mx2 = fmaxf(mx2, sacc0[8 + i]);
          mx3 = fmaxf(mx3, sacc1[8 + i]);
        }
        const float mx = pair_max32(fmaxf(fmaxf(mx0, mx1), fmaxf(mx2, mx3))) * c;
        const bool grow = mx > m_run + W;  // always true on the first tile (m_run = -inf)
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = grow ? ceilf(mx) : m_run;
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        }
        const float negm = -m_run;
        const f16x2 ones = {(__fp16)1.0f, (__fp16)1.0f};
        // the row sum in four independent chains, one per step (a single
        // chain of dependent adds would serialise the step's weights)
        float psum4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        // ---- weights for 16 keys at a time, each step feeding 4 PV MFMAs
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f32x16 &src = (s < 2) ? sacc0 : sacc1;
          bf16x8 pw, plo;
          f16x8 ph;
          if constexpr (EXACT) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float wv = fast_exp2(__builtin_fmaf(src[8 * (s & 1) + e], c, negm));
              pw[e] = (__bf16)wv;
              plo[e] = (__bf16)(wv - (float)pw[e]);
              psum4[s] += wv;
            }
          } else {
            // fp16 weights rounded toward zero (one packed conversion per
            // pair); the row sum adds the same rounded values, so the
            // rounding's common bias cancels in PV / l
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 8 * (s & 1) + 2 * e;
              const f16x2 pr = __builtin_amdgcn_cvt_pkrtz(fast_exp2(__builtin_fmaf(src[i], c, negm)),
                                                          fast_exp2(__builtin_fmaf(src[i + 1], c, negm)));
              ph[2 * e] = pr[0];
              ph[2 * e + 1] = pr[1];
              psum4[s] = __builtin_amdgcn_fdot2(pr, ones, psum4[s], false);
            }
          }
          // the step's V^T operands (2*DT transposing reads) before its MFMAs
          bf16x8 va[DT];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) va[dt] = vt_operand_at(sV + voff[dt] + s * 16 * D, 8 * D);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            if constexpr (EXACT) {
              oacc[dt] = mfma_bf16(va[dt], pw, oacc[dt]);
              oacc[dt] = mfma_bf16(va[dt], plo, oacc[dt]);
            } else {
              oacc[dt] = mfma_f16(__builtin_bit_cast(f16x8, va[dt]), ph, oacc[dt]);
            }
          }
        }
        l_run += (psum4[0] + psum4[1]) + (psum4[2] + psum4[3]);
      };
      if constexpr (S == 4) {
      // Two tiles per barrier: iteration k consumes tiles 2k and 2k+1 and,
      // before computing, copies 2k+2 and 2k+3 into the slots of 2k-2 and
      // 2k-1 (free once every wave has passed the barrier), so each copy has
      // a whole iteration to land.  A SIMD loaded on one tile and idle on the
      // other evens out within the pair.
      // the list entries of tiles t2 .. t2+3, read one iteration ahead so
      // that no LDS read stands between the barrier and the copies (entries
      // past U are never used)
      int ea = 0, eb = 0, ec = 0, ed = 0;
      if constexpr (FROM_LDS) {
        ea = slist[0]; eb = slist[1]; ec = slist[2]; ed = slist[3];
      }
      for (int t2 = 0; t2 < U; t2 += 2) {
        wait_vmcnt<0>();  // this wave's copies of tiles t2, t2+1
        barrier_lds();    // both visible to all waves; every wave is done with t2-2, t2-1
        int e0, e1;
        if constexpr (FROM_LDS) {
          e0 = ea;
          e1 = eb;
          if (t2 + 2 < U) issue_j(t2 + 2, __builtin_amdgcn_readfirstlane(ec & 0xffff));
          if (t2 + 3 < U) issue_j(t2 + 3, __builtin_amdgcn_readfirstlane(ed & 0xffff));
          ea = ec;
          eb = ed;
          ec = slist[t2 + 4];
          ed = slist[t2 + 5];
        } else {
          if (t2 + 2 < U) issue(t2 + 2);
          if (t2 + 3 < U) issue(t2 + 3);
          e0 = entry(t2);
          e1 = t2 + 1 < U ? entry(t2 + 1) : 0;
        }
        const bool m0 = active && ((e0 >> (16 + member)) & 1);
        const bool m1 = active && t2 + 1 < U && ((e1 >> (16 + member)) & 1);
        if (m0) tile(t2, e0);
        if (m1) tile(t2 + 1, e1);
      }
      } else {
      // One tile per barrier in a two-slot ring (half the LDS, so two
      // workgroups share a CU): iteration t consumes tile t and, right after
      // the barrier that frees the slot of tile t-1, copies tile t+1 into
      // it.  Tiles 0 and 1 come from the prologue.  Entries are read two
      // iterations ahead (entries past U are never used).
      static_assert(S == 2, "ring of two or four slots");
      int ecur = 0, enext = 0;
      if constexpr (FROM_LDS) {
        ecur = slist[0]; enext = slist[1];
      }
      for (int t = 0; t < U; ++t) {
        wait_vmcnt<0>();  // this wave's copies of tile t
        barrier_lds();    // visible to all waves; every wave is done with tile t-1
        int e;
        if constexpr (FROM_LDS) {
          e = ecur;
          if (t >= 1 && t + 1 < U) issue_j(t + 1, __builtin_amdgcn_readfirstlane(enext & 0xffff));
          ecur = enext;
          enext = slist[t + 2];
        } else {
          if (t >= 1 && t + 1 < U) issue(t + 1);
          e = entry(t);
        }
        if (active && ((e >> (16 + member)) & 1)) tile(t, e);
      }
      }
    };
    if (U <= LMAX) main_loop(std::integral_constant<bool, true>{});
    else main_loop(std::integral_constant<bool, false>{});
    const float l_tot = pair_sum32(l_run);
    const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= inv_l;
    // each row's log-sum-exp for the backward: from its recompute (the sparse
    // branch alone) or from a training forward
    if (args.lse && active && lane < 32 && n < args.n_tokens)
      args.lse[(int64_t)bh * args.nb * 64 + n] = m_run + log2f(l_tot);
    // a training forward also keeps O_s (fp32, the problem's strides; lane
    // holds dims 32*dt + 8*q4 + 4*g + 0..3 of row n), before the merge
    if (LOWRANK && args.os_save && active) {
      float *orow = args.os_save + base + n * args.stride_n;
      const bool valid = n < args.n_tokens;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v = {oacc[dt][4 * q4], oacc[dt][4 * q4 + 1], oacc[dt][4 * q4 + 2], oacc[dt][4 * q4 + 3]};
          if (!valid) v = f32x4{0.f, 0.f, 0.f, 0.f};
          *(f32x4 *)(orow + 32 * dt + 8 * q4 + 4 * g) = v;
        }
      }
    }
  }
  if (!active) return;
  attn_finish<D, LOWRANK, ACCUM, OUTF32>(args, qreg, oacc, n, base, bh, lane, sfreq);
  };  // run_group
  if constexpr (FALLBACK) {
    // the bf16 form as the fallback of the fp16 one: a grid of
    // bh_count x per_head workgroups, each taking every per_head-th group of
    // its head, and only for the flagged heads (so that the common case, no
    // head flagged, costs one flag read per workgroup)
    const int per_head = (int)(gridDim.x / args.bh_count);
    const int bh = (int)(blockIdx.x / per_head);
    if (!v_overflow(bh)) return;
    for (int64_t group = blockIdx.x % per_head; group < args.ngroups; group += per_head) {
      run_group(bh, group);
      __syncthreads();  // every wave done with the ring, list and table before the next group
    }
  } else {
  const int64_t L = blockIdx.x;
  const int64_t sidx = L / 8;
  const int64_t bh64 = sidx / args.groups_per_xcd;
  const int64_t group = (L % 8) * args.groups_per_xcd + sidx % args.groups_per_xcd;
  if (bh64 >= args.bh_count || group >= args.ngroups) return;
  run_group((int)bh64, group);
  }
}

// ---------------------------------------------------------------- k_quant8
// Per (batch, head, 64-token block): absmax of Q, K and V over the valid
// tokens; scale = fl32(absmax/448), inv = fl32(448/absmax) (1 and 1 for an
// all-zero block); codes = e4m3(fl32(x * inv)), padded rows 0.  Q gets its
// scales only (the attention kernel quantises the rows it holds); K and V
// codes are written as the block's tile image.  Grid (nb, B*H), 256
// threads: thread t holds dims [D/4*(t%4), +D/4) of token t/4.
template <int D>
__global__ __launch_bounds__(256) void k_quant8(Quant8Args a) {
  constexpr int PER = D / 4;
  __shared__ __attribute__((aligned(16))) uint8_t img[64 * D];
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.heads, h = bh % a.heads;
  const int64_t base = (int64_t)b * a.stride_b + (int64_t)h * a.stride_h;
  const int r = tid >> 2, part = tid & 3;
  const int64_t n = (int64_t)c * 64 + r;
  const bool valid = n < a.n_tokens;
  const int64_t roff = base + (valid ? n : 0) * a.stride_n + part * PER;

  auto load = [&](const uint16_t *X, float *x) {
#pragma unroll
    for (int i = 0; i < PER; i += 8) {
      const u32x4 w = *(const u32x4 *)(X + roff + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[i + 2 * e] = valid ? bflo(w[e]) : 0.0f;
        x[i + 2 * e + 1] = valid ? bfhi(w[e]) : 0.0f;
      }
    }
  };
  auto block_absmax = [&](const float *x) -> float {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return m;
  };
  const int64_t sidx = (int64_t)bh * a.nb + c;
  float x[PER];

  load(a.q, x);
  {
    const float m = block_absmax(x);
    if (tid == 0) {
      a.qsc[2 * sidx] = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
      a.qsc[2 * sidx + 1] = m > 0.0f ? __fdiv_rn(448.0f, m) : 1.0f;
    }
  }
  // K: codes of 8 consecutive dims are 8 consecutive image bytes
  load(a.k, x);
  {
    const float m = block_absmax(x);
    const float inv = m > 0.0f ? __fdiv_rn(448.0f, m) : 1.0f;
    if (tid == 0) a.ksc[sidx] = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
#pragma unroll
    for (int i = 0; i < PER; i += 8) {
      int w0 = cvt_fp8x2<false>(x[i] * inv, x[i + 1] * inv, 0);
      w0 = cvt_fp8x2<true>(x[i + 2] * inv, x[i + 3] * inv, w0);
      int w1 = cvt_fp8x2<false>(x[i + 4] * inv, x[i + 5] * inv, 0);
      w1 = cvt_fp8x2<true>(x[i + 6] * inv, x[i + 7] * inv, w1);
      *(uint2 *)(img + img_k_off<D>(r, part * PER + i)) = make_uint2((uint32_t)w0, (uint32_t)w1);
    }
  }
  // V: the codes of row r as fp16 values (0 past N)
  load(a.v, x);
  {
    const float m = block_absmax(x);
    const float inv = m > 0.0f ? __fdiv_rn(448.0f, m) : 1.0f;
    if (tid == 0) a.vsc[sidx] = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
    uint16_t *vrow = a.vh + ((int64_t)bh * a.nb * 64 + (int64_t)c * 64 + r) * D + part * PER;
#pragma unroll
    for (int i = 0; i < PER; i += 8) {
      int w0 = cvt_fp8x2<false>(x[i] * inv, x[i + 1] * inv, 0);
      w0 = cvt_fp8x2<true>(x[i + 2] * inv, x[i + 3] * inv, w0);
      int w1 = cvt_fp8x2<false>(x[i + 4] * inv, x[i + 5] * inv, 0);
      w1 = cvt_fp8x2<true>(x[i + 6] * inv, x[i + 7] * inv, w1);
      *(u32x4 *)(vrow + i) = e4m3x8_f16(make_uint2((uint32_t)w0, (uint32_t)w1));
    }
  }
  __syncthreads();
  u32x4 *dst = (u32x4 *)(a.kv8 + sidx * (64 * D));
#pragma unroll
  for (int i = tid; i < 4 * D; i += 256) dst[i] = *(const u32x4 *)(img + 16 * i);
}

// ------------------------------------------------------------------ k_attn8
// The sparse branch with e4m3 operands: S^T = K Q^T on
// v_mfma_f32_32x32x64_f8f6f4 (K codes from the block's K tile image, Q codes
// quantised in registers with the query block's inv scale), and O^T = V^T P^T
// on v_mfma_f32_32x32x16_f16 with fp16 weights against the V codes as fp16
// values (exact).  The workgroup shape, group walk, LDS ring and lazy softmax
// reference follow k_attn; a tile is the K image (64*D bytes, one contiguous
// copy) and the 64 V code rows (64*D fp16, the V-style chunk swizzle).  Per
// listed key block j (constants staged in LDS with the list):
//   logits (base 2)  t = acc * (sq * sk_j * scale * log2 e) - m_ref,
//   weights          P' = 2^(t + u_j) with u_j = 8 + log2(sv_j / sigma),
// sigma the largest V scale on the group's list, so P' * code_v carries the
// V scale; m_ref is an integer that moves (with an exact power-of-two
// rescale) only when a tile max exceeds it by more than 7, so P' < 2^15
// stays inside fp16.  Each weight is rounded once to fp16 (toward zero) and
// the row sum adds 2^-u_j times the same rounded weights.  Finally
// O = O' * sigma * 2^-8 / l.
template <int D, int G, int S, bool LOWRANK, bool ACCUM, bool OUTF32>
__global__ __launch_bounds__(128 * G) void k_attn8(AttnArgs args) {
  constexpr int P = kAttn8P;  // tiles per barrier
  constexpr int NS = D / 16;
  constexpr int DT = D / 32;
  constexpr int K8 = D / 64;            // fp8 k-steps over head_dim
  constexpr int NT = 128 * G;
  constexpr int CH = D / 8;              // 16-byte chunks per V row
  constexpr int KB = 64 * D;             // bytes of the K image
  constexpr int TB = KB + 128 * D;       // bytes per tile: K image, then 64 V rows of fp16
  constexpr int KC = KB / 16;             // 16-byte chunks of the K image
  constexpr int VOPS = 64 * CH / NT;      // V row chunks per thread
  constexpr int OPS = 1 + VOPS;           // DMA ops per thread per tile: one K chunk (thread t takes
                                          // chunk t % KC, so every wave counts the same ops), VOPS V chunks
  static_assert(VOPS >= 1 && (64 * CH) % NT == 0 && KC <= NT && NT % KC == 0, "tile split");
  static_assert(S >= 2 && S * OPS <= 63, "ring depth");
  constexpr int LMAX = kAttn8Lmax;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * TB];
  __shared__ int32_t slist[LMAX + 8];  // + room for the reads ahead past the end
  __shared__ float sck[LMAX], sku[LMAX], skw[LMAX];
  __shared__ float sred[2 * G];
  __shared__ __attribute__((aligned(16))) float sfreq[D / 2];  // rotary inverse frequency per pair

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int member = wave >> 1, half = wave & 1;
  const int64_t L = blockIdx.x;
  const int64_t sidx = L / 8;
  const int64_t bh64 = sidx / args.groups_per_xcd;
  const int64_t group = (L % 8) * args.groups_per_xcd + sidx % args.groups_per_xcd;
  if (bh64 >= args.bh_count || group >= args.ngroups) return;
  const int bh = (int)bh64;
  const int64_t gidx = (int64_t)bh * args.ngroups + group;
  const int qb = args.ugroup[gidx * G + member];
  const bool active = qb >= 0;
  const int b = bh / args.heads, h = bh % args.heads;
  const int64_t base = (int64_t)b * args.stride_b + (int64_t)h * args.stride_h;
  const int64_t n = (int64_t)(active ? qb : 0) * 64 + 32 * half + (lane & 31);

  const uint16_t *qrow = args.q + base + n * args.stride_n;
  bf16x8 qreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qreg[s] = *(const bf16x8 *)(qrow + 16 * s + 8 * g);
  const int64_t qs_idx = (int64_t)bh * args.nb + (active ? qb : 0);
  const float sq = args.qsc[2 * qs_idx], iq = args.qsc[2 * qs_idx + 1];
  const int32_t *list = args.ulist + gidx * args.list_stride;
  const int U = args.ucount[gidx];
  const float *ksc = args.ksc + (int64_t)bh * args.nb;
  const float *vsc = args.vsc + (int64_t)bh * args.nb;
  // sigma: the largest V scale on the list
  for (int p2 = tid; p2 < D / 2; p2 += NT) sfreq[p2] = rope_freq(2 * p2, args.rope);
  float vmax = 0.0f;
  for (int t = tid; t < U; t += NT) vmax = fmaxf(vmax, vsc[list[t] & 0xffff]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o, 64));
  if (lane == 0) sred[wave] = vmax;
  __syncthreads();
  float sigma = sred[0];
#pragma unroll
  for (int w = 1; w < 2 * G; ++w) sigma = fmaxf(sigma, sred[w]);
  const float log2_sigma = __log2f(sigma);
  const float c_scale = args.scale_log2e;
  auto consts = [&](int j, float &ck, float &ku, float &kw) {
    ck = ksc[j] * c_scale;
    // a V block far below sigma (tiny or denormal absmax) keeps a finite
    // weight 2^-ku; its codes times sigma-relative weights are negligible
    ku = fmaxf(8.0f + (__log2f(vsc[j]) - log2_sigma), -100.0f);
    kw = fast_exp2(-ku);
  };
  for (int t = tid; t < min(U, LMAX); t += NT) {
    const int ent = list[t];
    slist[t] = ent;
    consts(ent & 0xffff, sck[t], sku[t], skw[t]);
  }
  // Q codes: byte e of k-step s holds dim 64s + 16(e/8) + 8g + e%8, i.e.
  // element e%8 of qreg[4s + e/8]
  i32x8 q8[K8];
  if (args.q8) {
    // pre-quantised input: the caller's codes, in the same byte order
    const uint8_t *qc = args.q8 + base + n * args.stride_n;
#pragma unroll
    for (int s8 = 0; s8 < K8; ++s8) {
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint2 u = *(const uint2 *)(qc + 64 * s8 + 16 * pr + 8 * g);
        q8[s8][2 * pr] = (int)u.x;
        q8[s8][2 * pr + 1] = (int)u.y;
      }
    }
  } else {
#pragma unroll
    for (int s8 = 0; s8 < K8; ++s8) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const bf16x8 &src = qreg[4 * s8 + (w >> 1)];
        const int e0 = 4 * (w & 1);
        int v = cvt_fp8x2<false>((float)src[e0] * iq, (float)src[e0 + 1] * iq, 0);
        v = cvt_fp8x2<true>((float)src[e0 + 2] * iq, (float)src[e0 + 3] * iq, v);
        q8[s8][w] = v;
      }
    }
  }
  wait_vmcnt<0>();  // Q, scales and the list in registers before the tile copies start
  __syncthreads();

  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  // per-lane LDS offsets of the MFMA operands inside a tile: K image bytes;
  // V^T transposed-read rows 4g + (l%16)/4 (+16 per 16-key step, +8 for the
  // second half), dims 32dt + 16((l/16)%2) + 4(l%4), in fp16 elements from
  // the V part
  int koff[K8][2], voff[DT];
#pragma unroll
  for (int s8 = 0; s8 < K8; ++s8) {
    const int r = lane & 31;
    const int f = (r / (256 / D)) & (D / 16 - 1);
    const int c0 = 4 * s8 + 2 * g;
    koff[s8][0] = r * D + ((c0 ^ f) << 4);
    koff[s8][1] = r * D + (((c0 + 1) ^ f) << 4);
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int i = lane & 15, dhalf = (lane >> 4) & 1;
    const int dstart = 32 * dt + 16 * dhalf + 4 * (i & 3);
    const int r0 = 4 * g + (i >> 2);
    voff[dt] = r0 * D + (((dstart >> 3) ^ swz_v<D>(r0)) << 3) + (dstart & 7);
  }
  // this thread's source byte offsets: its K image chunk, and its V row chunks
  // (row-major, V-style swizzle) inside a block
  const uint32_t gk = (uint32_t)((tid % KC) * 16);
  uint32_t gv[VOPS];
#pragma unroll
  for (int o = 0; o < VOPS; ++o) {
    const int cidx = o * NT + tid, row = cidx / CH, pc = cidx % CH;
    gv[o] = (uint32_t)((row * D + ((pc ^ swz_v<D>(row)) * 8)) * 2);
  }
  auto ld16 = [](const uint8_t *p) -> u32x4 { return *(const u32x4 *)p; };
  auto cat = [](u32x4 a, u32x4 b) -> i32x8 {
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  };
  const uint8_t *img = args.kv8 + (int64_t)bh * args.nb * KB;
  const uint16_t *vcodes = args.vh + (int64_t)bh * args.nb * 64 * D;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  auto main_loop = [&](auto lds_tag) {
    constexpr bool FROM_LDS = decltype(lds_tag)::value;
    auto entry = [&](int t) __attribute__((always_inline)) -> int {
      if constexpr (FROM_LDS) return slist[t];
      else return list[t];
    };
    auto issue_j = [&](int t, int j) {
      j = __builtin_amdgcn_readfirstlane(j);
      const uint32_t m0 = ring_lds + (uint32_t)((t % S) * TB);
      // K image: chunk t % KC at its own position (waves past KC/64 repeat
      // the first waves' chunks, the same bytes to the same place)
      lds_dma16_m0(img + (int64_t)j * KB, gk, m0 + (uint32_t)(((wave_s * 64) % KC) * 16));
      const uint16_t *vj = vcodes + (int64_t)j * 64 * D;
#pragma unroll
      for (int o = 0; o < VOPS; ++o)
        lds_dma16_m0(vj, gv[o], m0 + (uint32_t)KB + (uint32_t)((o * NT + wave_s * 64) * 16));
    };
    auto issue = [&](int t) { issue_j(t, entry(t) & 0xffff); };
    // P tiles per barrier in an S-slot ring (S/P groups of slots): group k
    // (tiles kP .. kP+P-1) is consumed while the next S/P-1 groups are in
    // flight; group k+S/P-1 is copied into the slots of group k-1 right after
    // the barrier that frees them, before the compute.
    constexpr int NGR = S / P;
    static_assert(S % P == 0 && NGR >= 2, "ring of whole groups");
    for (int t = 0; t < (NGR - 1) * P; ++t)
      if (t < U) issue(t);
    // one listed tile t (list entry ent) for this wave's 32 query rows
    auto walk_tile = [&](int t, int ent) __attribute__((always_inline)) {
      float ck, ku, kw;
      if constexpr (FROM_LDS) {
        ck = sck[t]; ku = sku[t]; kw = skw[t];
      } else {
        consts(ent & 0xffff, ck, ku, kw);
      }
      const int j = ent & 0xffff;
      const uint8_t *tile = ring + (t % S) * TB;
      f32x16 sacc0 = f32x16{}, sacc1 = f32x16{};
#pragma unroll
      for (int s8 = 0; s8 < K8; ++s8) {
        sacc0 = mfma_fp8(cat(ld16(tile + koff[s8][0]), ld16(tile + koff[s8][1])), q8[s8], sacc0);
        sacc1 = mfma_fp8(cat(ld16(tile + koff[s8][0] + 32 * D), ld16(tile + koff[s8][1] + 32 * D)),
                         q8[s8], sacc1);
      }
      if ((int64_t)(j + 1) * 64 > args.n_tokens) {
        const int lim = (int)(args.n_tokens - (int64_t)j * 64) - 4 * g;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kc = 8 * (i >> 2) + (i & 3);
          if (kc >= lim) sacc0[i] = -INFINITY;
          if (kc + 32 >= lim) sacc1[i] = -INFINITY;
        }
      }
      const float c = sq * ck;
      // the tile max in four independent chains
      float mx0 = -INFINITY, mx1 = -INFINITY, mx2 = -INFINITY, mx3 = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mx0 = fmaxf(mx0, sacc0[i]);
        mx1 = fmaxf(mx1, sacc1[i]);
        mx2 = fmaxf(mx2, sacc0[8 + i]);
        mx3 = fmaxf(mx3, sacc1[8 + i]);
      }
      const float mx = pair_max32(fmaxf(fmaxf(mx0, mx1), fmaxf(mx2, mx3))) * c;
      const bool grow = mx > m_run + 7.0f;  // always true on the first tile (m_run = -inf)
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? ceilf(mx) : m_run;
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      }
      // fp16 weights rounded toward zero (one packed conversion per pair),
      // 16 keys per step, each step feeding DT PV MFMAs; the row sum, in four
      // independent chains, adds the same rounded weights
      const float off = ku - m_run;
      const f16x2 ones = {(__fp16)1.0f, (__fp16)1.0f};
      const uint16_t *sV = (const uint16_t *)(tile + KB);
      float psum4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f32x16 &src = (s < 2) ? sacc0 : sacc1;
        f16x8 ph;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 8 * (s & 1) + 2 * e;
          const f16x2 pr = __builtin_amdgcn_cvt_pkrtz(fast_exp2(__builtin_fmaf(src[i], c, off)),
                                                      fast_exp2(__builtin_fmaf(src[i + 1], c, off)));
          ph[2 * e] = pr[0];
          ph[2 * e + 1] = pr[1];
          psum4[s] = __builtin_amdgcn_fdot2(pr, ones, psum4[s], false);
        }
        bf16x8 va[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) va[dt] = vt_operand_at(sV + voff[dt] + s * 16 * D, 8 * D);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma_f16(__builtin_bit_cast(f16x8, va[dt]), ph, oacc[dt]);
      }
      l_run = __builtin_fmaf((psum4[0] + psum4[1]) + (psum4[2] + psum4[3]), kw, l_run);
    };
    if constexpr (FROM_LDS && P == 2 && NGR == 2) {
      // the list entries of tiles t2 .. t2+3, read one iteration ahead so
      // that no LDS read stands between the barrier and the copies (entries
      // past U are never used)
      int ea = slist[0], eb = slist[1], ec = slist[2], ed = slist[3];
      for (int t2 = 0; t2 < U; t2 += 2) {
        wait_vmcnt<0>();  // this wave's copies of tiles t2, t2+1
        barrier_lds();    // both visible to all waves; every wave is done with t2-2, t2-1
        const int e0 = ea, e1 = eb;
        if (t2 + 2 < U) issue_j(t2 + 2, ec & 0xffff);
        if (t2 + 3 < U) issue_j(t2 + 3, ed & 0xffff);
        ea = ec;
        eb = ed;
        ec = slist[t2 + 4];
        ed = slist[t2 + 5];
        if (active && ((e0 >> (16 + member)) & 1)) walk_tile(t2, e0);
        if (active && t2 + 1 < U && ((e1 >> (16 + member)) & 1)) walk_tile(t2 + 1, e1);
      }
    } else {
    for (int t2 = 0; t2 < U; t2 += P) {
      // tiles t2 .. t2+P-1 complete; the tiles copied after them (up to
      // t2 + (NGR-1)*P - 1) may be in flight
      wait_tiles<OPS, (NGR - 2) * P>(min((NGR - 2) * P, U - (t2 + P)));
      barrier_lds();
      uint32_t mm = 0;  // this wave's membership over the group
#pragma unroll
      for (int u = 0; u < P; ++u)
        if (t2 + u < U && active && ((entry(t2 + u) >> (16 + member)) & 1)) mm |= 1u << u;
      const int tn = t2 + (NGR - 1) * P;  // first tile of the group to copy now
      for (int u = 0; u < P; ++u)
        if (tn + u < U) issue(tn + u);
      if (!mm) continue;
      for (int t = t2; t < min(t2 + P, U); ++t) {
      if (!((mm >> (t - t2)) & 1)) continue;
      walk_tile(t, entry(t));
      }
    }
    }
  };
  if (U <= LMAX) main_loop(std::integral_constant<bool, true>{});
  else main_loop(std::integral_constant<bool, false>{});
  const float l_tot = pair_sum32(l_run);
  const float fin = l_tot > 0.0f ? sigma * 0.00390625f / l_tot : 0.0f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] *= fin;
  if (!active) return;
  // the bf16 Q rows are loaded again for the low-rank apply rather than held
  // in registers through the loop
  bf16x8 qlr[NS];
  if (LOWRANK) {
#pragma unroll
    for (int s = 0; s < NS; ++s) qlr[s] = *(const bf16x8 *)(qrow + 16 * s + 8 * g);
  }
  attn_finish<D, LOWRANK, ACCUM, OUTF32>(args, qlr, oacc, n, base, bh, lane, sfreq);
}

// ------------------------------------------------------------ k_mfma_probe
// Four independent MFMA chains per wave on constant operands (measurement of
// the sustained matrix-core rate); lane 0 of wave 0 keeps one result alive.
template <bool FP8>
__global__ __launch_bounds__(256) void k_mfma_probe(int iters, float *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  f32x16 a0 = f32x16{}, a1 = f32x16{}, a2 = f32x16{}, a3 = f32x16{};
  if constexpr (FP8) {
    const i32x8 x = {0x38383838 + lane, 0x30303030, 0x38383838, 0x30303030,
                     0x38383838, 0x30303030, 0x38383838, 0x30303030};
    for (int i = 0; i < iters; ++i) {
      a0 = mfma_fp8(x, x, a0);
      a1 = mfma_fp8(x, x, a1);
      a2 = mfma_fp8(x, x, a2);
      a3 = mfma_fp8(x, x, a3);
    }
  } else {
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (__bf16)(0.001f * (float)(lane + e));
    for (int i = 0; i < iters; ++i) {
      a0 = mfma_bf16(x, x, a0);
      a1 = mfma_bf16(x, x, a1);
      a2 = mfma_bf16(x, x, a2);
      a3 = mfma_bf16(x, x, a3);
    }
  }
  const float r = a0[0] + a1[1] + a2[2] + a3[3];
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) sink[blockIdx.x] = r;
  if (blockIdx.x == 0 && threadIdx.x == 0) {  // core-clock and reference-clock ticks of this wave
    sink[1024] = (float)(c1 - c0);
    sink[1025] = (float)(r1 - r0);
  }
}

void launch_mfma_probe(bool fp8, int iters, int blocks, float *sink, hipStream_t st) {
  if (fp8) hipLaunchKernelGGL(k_mfma_probe<true>, dim3(blocks), dim3(256), 0, st, iters, sink);
  else hipLaunchKernelGGL(k_mfma_probe<false>, dim3(blocks), dim3(256), 0, st, iters, sink);
}

// ---------------------------------------------------------------- launchers
void launch_setup(const SetupArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(k_setup, dim3((32 * a.D + 255) / 256), dim3(256), 0, st, a.wq, a.wk, a.D, a.rank,
                     a.wqT, a.wkT);
}

template <int D>
static void pass1_d(const Pass1Args &a, int nchunks, int bh, bool pool, bool state, bool quant,
                    hipStream_t st) {
  dim3 grid(nchunks, bh), block(256);
  const bool blk = a.blk_state != nullptr;
  const bool vh = a.vh != nullptr && !quant;
  if (pool && state && quant) {
    if (blk) hipLaunchKernelGGL((k_pass1<D, true, true, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_pass1<D, true, true, true, false>), grid, block, 0, st, a);
  } else if (pool && state && vh) {
    if (blk) hipLaunchKernelGGL((k_pass1<D, true, true, false, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_pass1<D, true, true, false, false, true>), grid, block, 0, st, a);
  } else if (pool && state) {
    if (blk) hipLaunchKernelGGL((k_pass1<D, true, true, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_pass1<D, true, true, false, false>), grid, block, 0, st, a);
  } else if (!pool && !state && vh) {
    hipLaunchKernelGGL((k_pass1<D, false, false, false, false, true>), grid, dim3(128), 0, st, a);
  } else if (pool) {
    hipLaunchKernelGGL((k_pass1<D, true, false, false, false>), grid, block, 0, st, a);
  } else {
    hipLaunchKernelGGL((k_pass1<D, false, true, false, false>), grid, block, 0, st, a);
  }
}

void launch_pass1(const Pass1Args &a, int D, int nchunks, int bh, bool pool, bool state, bool quant,
                  hipStream_t st) {
  if (D == 64) pass1_d<64>(a, nchunks, bh, pool, state, quant, st);
  else pass1_d<128>(a, nchunks, bh, pool, state, quant, st);
}

void launch_state_reduce(const float *part, int np, int D, int rank, int bh, uint16_t *st_out,
                         float *z, float *s32, hipStream_t st) {
  hipLaunchKernelGGL(k_state_reduce, dim3((D * 32 + 32 + 255) / 256, bh), dim3(256), 0, st, part, np, D,
                     rank, st_out, z, s32);
}

void launch_blk_partial(const uint8_t *blk, int nb, int parts, int D, int bh, float *part, hipStream_t st) {
  const int per = (nb + parts - 1) / parts;
  const dim3 grid((unsigned)parts, (unsigned)bh);
  if (D == 64) hipLaunchKernelGGL(k_blk_partial<64>, grid, dim3(256), 0, st, blk, nb, per, part);
  else hipLaunchKernelGGL(k_blk_partial<128>, grid, dim3(256), 0, st, blk, nb, per, part);
}

void launch_complement(const CompArgs &a, int D, hipStream_t st) {
  const dim3 grid((unsigned)(8 * a.groups_per_xcd * a.bh_count)), block(256);
  if (D == 64) hipLaunchKernelGGL((k_complement<64, kAttnG>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_complement<128, kAttnG>), grid, block, 0, st, a);
}

void launch_scores(const float *qp, const float *kp, float *s, int nb, int D, int bh,
                   hipStream_t st) {
  dim3 grid((nb + 63) / 64, (nb + 63) / 64, bh);
  if (D == 64) hipLaunchKernelGGL(k_scores<64>, grid, dim3(256), 0, st, qp, kp, s, nb);
  else hipLaunchKernelGGL(k_scores<128>, grid, dim3(256), 0, st, qp, kp, s, nb);
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

void launch_schedule(const int32_t *map, int nb, int kb, int G, int ngroups, int list_stride,
                     int bh, int32_t *ugroup, int32_t *ucount, int32_t *ulist, hipStream_t st) {
  hipLaunchKernelGGL(k_order, dim3((nb + kOrderPer - 1) / kOrderPer, bh), dim3(1024), (size_t)nb * 4, st, map, nb,
                     kb, G, ngroups, ugroup);
  if (kb > 0 && kb <= kGroupMaxKb && kGroupWin % G == 0) {
    const dim3 grid((ngroups * G + kGroupWin - 1) / kGroupWin, bh), block(64);
    const size_t lds = (size_t)(nb + 31) / 32 * 4;
    if (kb <= 16) hipLaunchKernelGGL(k_group<16>, grid, block, lds, st, map, nb, kb, G, ngroups, ugroup);
    else if (kb <= 32) hipLaunchKernelGGL(k_group<32>, grid, block, lds, st, map, nb, kb, G, ngroups, ugroup);
    else if (kb <= 48) hipLaunchKernelGGL(k_group<48>, grid, block, lds, st, map, nb, kb, G, ngroups, ugroup);
    else hipLaunchKernelGGL(k_group<64>, grid, block, lds, st, map, nb, kb, G, ngroups, ugroup);
  }
  if (kb > 0) {
    const size_t lds = (size_t)kUnionWaves * ((nb + 3) / 4) * 4;
    hipLaunchKernelGGL(k_union, dim3((ngroups + kUnionWaves - 1) / kUnionWaves, bh), dim3(64 * kUnionWaves), lds,
                       st, map, nb, kb, G, ngroups, list_stride, ugroup, ucount, ulist);
  }
}

constexpr int64_t kFallbackPerHead = 32;  // workgroups per head of the bf16 fallback launch
// fp32 output: the EXACT form.  bf16 output with the sparse branch: the fp16
// form, then the EXACT form for the heads whose fp16 V copy is flagged (an
// empty pass, each workgroup reading its head's flags, when none is).
template <int D, int G, int S, bool SPARSE, bool LOWRANK, bool ACCUM>
static void attn_d3(const AttnArgs &a, bool outf32, hipStream_t st) {
  dim3 grid((unsigned)(8 * a.groups_per_xcd * a.bh_count)), block(128 * G);
  if (outf32) {
    hipLaunchKernelGGL((k_attn<D, G, S, SPARSE, LOWRANK, ACCUM, true, true>), grid, block, 0, st, a);
  } else if constexpr (!SPARSE) {
    hipLaunchKernelGGL((k_attn<D, G, S, SPARSE, LOWRANK, ACCUM, false, false>), grid, block, 0, st, a);
  } else {
    hipLaunchKernelGGL((k_attn<D, G, S, SPARSE, LOWRANK, ACCUM, false, false>), grid, block, 0, st, a);
    // the fallback: per_head workgroups per head, each looping over groups
    const int64_t per_head = std::min<int64_t>(a.ngroups, kFallbackPerHead);
    hipLaunchKernelGGL((k_attn<D, G, S, SPARSE, LOWRANK, ACCUM, false, true, true>),
                       dim3((unsigned)(per_head * a.bh_count)), block, 0, st, a);
  }
}

template <int D, int G, int S, bool SPARSE, bool LOWRANK>
static void attn_d2(const AttnArgs &a, bool accum, bool outf32, hipStream_t st) {
  if (accum) attn_d3<D, G, S, SPARSE, LOWRANK, true>(a, outf32, st);
  else attn_d3<D, G, S, SPARSE, LOWRANK, false>(a, outf32, st);
}

template <int D, int G, int S>
static void attn_d(const AttnArgs &a, bool sparse, bool lowrank, bool accum, bool outf32,
                   hipStream_t st) {
  if (sparse && lowrank) attn_d2<D, G, S, true, true>(a, accum, outf32, st);
  else if (sparse) attn_d2<D, G, S, true, false>(a, accum, outf32, st);
  else attn_d2<D, G, S, false, true>(a, accum, outf32, st);
}

int attn_group_size() { return kAttnG; }

void launch_attn(const AttnArgs &a, int D, bool sparse, bool lowrank, bool accum, bool outf32,
                 hipStream_t st) {
  if (D == 64) attn_d<64, kAttnG, kAttnS>(a, sparse, lowrank, accum, outf32, st);
  else attn_d<128, kAttnG, kAttnS>(a, sparse, lowrank, accum, outf32, st);
}

// Pre-quantised input: the caller's e4m3 codes of K and V laid out as the
// block's tile image (rows at or past N as code 0) and the caller's scales
// copied; Q keeps its scale only (the attention kernel loads its Q codes).
// Same grid and thread mapping as k_quant8.
template <int D>
__global__ __launch_bounds__(256) void k_image8(Quant8Args a) {
  constexpr int C8 = D / 8;             // 8-code chunks per row
  constexpr int IT = 64 * C8 / 256;     // chunks per thread and tensor
  __shared__ __attribute__((aligned(16))) uint8_t img[64 * D];
  const int tid = threadIdx.x;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.heads, h = bh % a.heads;
  const int64_t base = (int64_t)b * a.stride_b + (int64_t)h * a.stride_h;
  const int64_t sidx = (int64_t)bh * a.nb + c;
  if (tid == 0) {
    a.qsc[2 * sidx] = a.qs_in[sidx];
    a.qsc[2 * sidx + 1] = 1.0f;  // no Q quantisation on this path
    a.ksc[sidx] = a.ks_in[sidx];
    a.vsc[sidx] = a.vs_in[sidx];
  }
  // chunk i = it*256 + tid is codes 8*(i % C8) .. +7 of row i / C8, so that
  // neighbouring lanes read and write neighbouring 8-code chunks of a row
  uint2 kw[IT], vw[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = it * 256 + tid, r = i / C8, d0 = 8 * (i % C8);
    const int64_t n = (int64_t)c * 64 + r;
    const bool valid = n < a.n_tokens;
    const int64_t off = base + (valid ? n : 0) * a.stride_n + d0;
    kw[it] = valid ? *(const uint2 *)(a.k8 + off) : make_uint2(0u, 0u);
    vw[it] = valid ? *(const uint2 *)(a.v8 + off) : make_uint2(0u, 0u);
  }
  // K: 8 consecutive dims are 8 consecutive image bytes
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = it * 256 + tid;
    *(uint2 *)(img + img_k_off<D>(i / C8, 8 * (i % C8))) = kw[it];
  }
  // V: the codes of each row as fp16 values (0 past N)
  uint16_t *vblk = a.vh + ((int64_t)bh * a.nb * 64 + (int64_t)c * 64) * D;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int i = it * 256 + tid;
    *(u32x4 *)(vblk + (i / C8) * D + 8 * (i % C8)) = e4m3x8_f16(vw[it]);
  }
  __syncthreads();
  u32x4 *dst = (u32x4 *)(a.kv8 + sidx * (64 * D));
#pragma unroll
  for (int i = tid; i < 4 * D; i += 256) dst[i] = *(const u32x4 *)(img + 16 * i);
}

void launch_quant8(const Quant8Args &a, int D, int bh, hipStream_t st) {
  dim3 grid(a.nb, bh), block(256);
  if (a.k8) {
    if (D == 64) hipLaunchKernelGGL(k_image8<64>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(k_image8<128>, grid, block, 0, st, a);
    return;
  }
  if (D == 64) hipLaunchKernelGGL(k_quant8<64>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(k_quant8<128>, grid, block, 0, st, a);
}

template <int D, int G, int S, bool LOWRANK>
static void attn8_d2(const AttnArgs &a, bool accum, bool outf32, hipStream_t st) {
  dim3 grid((unsigned)(8 * a.groups_per_xcd * a.bh_count)), block(128 * G);
  if (accum) {
    if (outf32) hipLaunchKernelGGL((k_attn8<D, G, S, LOWRANK, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn8<D, G, S, LOWRANK, true, false>), grid, block, 0, st, a);
  } else {
    if (outf32) hipLaunchKernelGGL((k_attn8<D, G, S, LOWRANK, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn8<D, G, S, LOWRANK, false, false>), grid, block, 0, st, a);
  }
}

void launch_attn8(const AttnArgs &a, int D, bool lowrank, bool accum, bool outf32, hipStream_t st) {
  if (D == 64) {
    if (lowrank) attn8_d2<64, kAttnG, kAttn8S, true>(a, accum, outf32, st);
    else attn8_d2<64, kAttnG, kAttn8S, false>(a, accum, outf32, st);
  } else {
    if (lowrank) attn8_d2<128, kAttnG, kAttn8S, true>(a, accum, outf32, st);
    else attn8_d2<128, kAttnG, kAttn8S, false>(a, accum, outf32, st);
  }
}

}  // namespace rola
