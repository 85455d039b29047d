// rola_backward.hip -- gfx950 kernels of the RoLA backward (training).
//
// Gradients of O = O_sparse + g * O_lr with respect to Q, K, V, the two
// low-rank projections and the output gate (pages: "SparkDiffusion: 265x
// Faster Video Generation on Consumer GPUs via Sparse Attention &
// Distillation", section "RoLA: Preserving Global Context at Extreme
// Sparsity"; README "AlibabaResearch/SparkDiffusion", sparse-finetune and
// distillation sections, which train the module and name its trainable
// projections and gate).  The block map is a constant of the backward: the
// top-k selection is piecewise constant in Q and K.
//
// Per (batch, head), with c = scale and L = O_lr:
//   sparse:   P = exp2(c log2e q.k - lse2), D_n = dO_n . O_s,n,
//             dS = P (dO.v - D), dq = c dS k, dk = c dS^T q, dv = P^T dO
//   low rank: a = phi(u), u = Wq^T R(q); num = S^T a, den = a.z, L = num/den;
//             with the gate g = sigmoid(y), y = q.w + b:
//             dg = dO.L, dy = dg g (1-g), dnum = g dO / den, dden = -g dg / den,
//             da = S dnum + z dden, du = da phi'(u), dq += R^T(Wq du) + dy w,
//             dWq = sum R(q) du^T, dS = sum a dnum^T, dz = sum a dden,
//             db = dS v + dz, dv += dS^T b, dw' = db phi'(Wk^T R(k)),
//             dk += R^T(Wk dw'), dWk = sum R(k) dw'^T, dw = sum dy q, db_gate = sum dy.
//
// Kernels, in launch order (after pass 1's state and a sparse-only forward
// with fp32 weights that leaves O_s and the row log-sum-exp, consistent with
// each other to about 16 bits, so that the P of the backward sums to one and
// D = dO . O_s = sum P dP -- with bf16 weights the sum of dS over a row's keys
// would not vanish and the error would show in dq):
//   k_bwd_prep   bf16 operand copies: Wq, Wk rank-permuted, S with d permuted
//   k_bwd_query  per query token: the low-rank and gate terms of dq, dL/du,
//                g a / den, dO in bf16 and D_n = dO . O_s (MFMA on 32-token tiles)
//   k_bwd_outer  sums X^T Y over tokens on MFMA (dS, dWq, dWk, gate weights)
//   k_bwd_sum, k_bwd_sum_heads  fixed-order sums of the partials
//   k_bwd_dz     dz and the gate bias gradient per head
//   k_bwd_dsops  bf16 operand copies of dS
//   k_bwd_key    per key token: the low-rank terms of dk, dv and dL/dw'
//   k_bwd_dq     sparse dq over each query block's kept key blocks
//   k_bwd_mapbits, k_bwd_tmap  query blocks that keep each key block
//   k_bwd_dkv    sparse dk, dv over the query blocks keeping each key block
#include "rola_device.h"

namespace rola {

// ------------------------------------------------------------ k_bwd_prep
// y = 0: Wq, Wk as bf16 [D][32] with the rank index permuted per 16-group
// (the A operand of R^T-side products whose B operand is an accumulator);
// y = 1: per head, S as a bf16 pair hi + lo, [32][D] each with d permuted
// per 16-group (the A operand of S dnum).  Ranks >= rank are zero.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_prep(BwdArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.y == 0) {
    if (t >= D * 32) return;
    const int d = (int)(t / 32), pos = (int)(t % 32), r = perm16_key_of_pos(pos);
    const float wq = r < a.rank ? a.wq[d * a.rank + r] : 0.0f;
    const float wk = r < a.rank ? a.wk[d * a.rank + r] : 0.0f;
    a.wqP[t] = __builtin_bit_cast(uint16_t, (__bf16)wq);
    a.wkP[t] = __builtin_bit_cast(uint16_t, (__bf16)wk);
  } else {
    if (t >= a.bh_count * 32 * D) return;
    const int64_t bh = t / (32 * D);
    const int r = (int)((t / D) % 32), p = (int)(t % D), d = perm16_key_of_pos(p);
    const float x = a.s32[bh * D * 32 + d * 32 + r];
    const __bf16 hi = (__bf16)x;
    a.sd[t] = __builtin_bit_cast(uint16_t, hi);
    a.sd[a.bh_count * 32 * D + t] = __builtin_bit_cast(uint16_t, (__bf16)(x - (float)hi));
  }
}

// inverse rotation (R^T) of the pair (x0, x1) at even dim d of a token at (pt, ph, pw)
static __device__ __forceinline__ void rope_back(float &x0, float &x1, int d, int pt, int ph, int pw,
                                                 float freq, const RopeArgsDev &ra) {
  const int pos = d < ra.off1 ? pt : (d < ra.off2 ? ph : pw);
  float rev = (float)pos * freq * 0.15915494309189535f;
  rev = rev - floorf(rev);
  const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
  const float y0 = x0 * cs + x1 * sn, y1 = x1 * cs - x0 * sn;
  x0 = y0;
  x1 = y1;
}

// x as hi + lo, both bf16 (hi = RNE(x), lo = RNE(x - hi)), into element e of two operands
static __device__ __forceinline__ void split_bf16(float x, bf16x8 &hi, bf16x8 &lo, int e) {
  const __bf16 h = (__bf16)x;
  hi[e] = h;
  lo[e] = (__bf16)(x - (float)h);
}

static __device__ __forceinline__ uint2 pack_bf16x4(float v0, float v1, float v2, float v3) {
  const __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1, b2 = (__bf16)v2, b3 = (__bf16)v3;
  uint2 o;
  o.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
  o.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
  return o;
}

// ----------------------------------------------------------- k_bwd_query
// One wave per 32-token tile of one (batch, head); lane column t = token.
// MFMA C/D rows are the rank index (u, a, da, du) or the head dim (num, dO,
// dRq) in the accumulator order 8*(i/4) + 4*g + i%4, so the elementwise
// steps are lane-local and the bf16 accumulators feed the next product as B
// operands against the permuted A copies.
template <int D, bool GATE, bool DF32>
__global__ __launch_bounds__(256) void k_bwd_query(BwdArgs a) {
  constexpr int NS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) float sfreq[D / 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, col = lane & 31;
  for (int p2 = tid; p2 < D / 2; p2 += 256) sfreq[p2] = rope_freq(2 * p2, a.rope);
  __syncthreads();
  const int bh = blockIdx.y;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= 2 * a.nb) return;
  const int b = bh / a.heads, h = bh % a.heads;
  const int64_t base = (int64_t)b * a.stride_b + (int64_t)h * a.stride_h;
  const int64_t n_pad = (int64_t)a.nb * 64;
  const int64_t n = (int64_t)tile * 32 + col;
  const bool valid = n < a.n_tokens;
  const int64_t nc = valid ? n : a.n_tokens - 1;
  const int64_t row = (int64_t)bh * n_pad + n;

  bf16x8 qreg[NS];
  const uint16_t *qrow = a.q + base + nc * a.stride_n;
#pragma unroll
  for (int s = 0; s < NS; ++s) qreg[s] = *(const bf16x8 *)(qrow + 16 * s + 8 * g);
  float y = 0.0f;
  if (GATE) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 w0 = *(const f32x4 *)(a.gate + 16 * s + 8 * g);
      const f32x4 w1 = *(const f32x4 *)(a.gate + 16 * s + 8 * g + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y += (float)qreg[s][e] * w0[e];
        y += (float)qreg[s][4 + e] * w1[e];
      }
    }
    y += shfl_xor32(y);
    y += a.gate[D];
  }
  // u = Wq^T R(q), a = phi(u), den = a . z
  int pt, ph, pw;
  token_pos(nc, a.rope, pt, ph, pw);
  f32x16 uacc = f32x16{};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const f32x4 fr = *(const f32x4 *)&sfreq[8 * s + 4 * g];
    const float freq[4] = {fr[0], fr[1], fr[2], fr[3]};
    const bf16x8 qr = rope8(qreg[s], 16 * s + 8 * g, pt, ph, pw, freq, a.rope);
    uacc = mfma_bf16(*(const bf16x8 *)(a.wqT + col * D + 16 * s + 8 * g), qr, uacc);
  }
  // the state this token's low-rank term reads: the head's, or (complement
  // scope) its query block's
  const int64_t qi = (int64_t)bh * a.nb + (tile >> 1);
  const f32x4 *zb = (const f32x4 *)(a.comp ? a.zc + qi * 32 : a.z + (int64_t)bh * 32);
  f32x4 zr[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) zr[q4] = zb[2 * q4 + g];  // z[8 q4 + 4 g .. +4]
  float av[16];
  float den = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + 4 * g + (i & 3);
    av[i] = r < a.rank ? phi(uacc[i]) : 0.0f;
    den += av[i] * zr[i >> 2][i & 3];
  }
  den += shfl_xor32(den);
  // den = 0 only for an empty complement (every block kept): no low-rank term
  const float inv_den = den > 0.0f ? 1.0f / den : 0.0f;
  bf16x8 aop[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) aop[i >> 3][i & 7] = (__bf16)av[i];
  // num = S^T a (rows d)
  const uint16_t *stb = a.comp ? a.stc + qi * D * 32 : a.st + (int64_t)bh * D * 32;
  f32x16 num[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    num[dt] = f32x16{};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      num[dt] = mfma_bf16(*(const bf16x8 *)(stb + (32 * dt + col) * 32 + 16 * s2 + 8 * g), aop[s2], num[dt]);
  }
  // dO and O_s at the lane's dims d = 32 dt + 8 q4 + 4 g + j; D_n and dg
  f32x16 dov[DT];
  float dn_p = 0.0f, dg_p = 0.0f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      float dv4[4];
      if (DF32) {
        const f32x4 x = *(const f32x4 *)((const float *)a.dout + base + nc * a.stride_n + d0);
#pragma unroll
        for (int j = 0; j < 4; ++j) dv4[j] = valid ? x[j] : 0.0f;
      } else {
        const uint2 u = *(const uint2 *)((const uint16_t *)a.dout + base + nc * a.stride_n + d0);
        dv4[0] = bflo(u.x); dv4[1] = bfhi(u.x); dv4[2] = bflo(u.y); dv4[3] = bfhi(u.y);
#pragma unroll
        for (int j = 0; j < 4; ++j) dv4[j] = valid ? dv4[j] : 0.0f;
      }
      const f32x4 o4 = *(const f32x4 *)(a.os + base + n * a.stride_n + d0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dov[dt][4 * q4 + j] = dv4[j];
        dn_p += dv4[j] * o4[j];
        dg_p += dv4[j] * (num[dt][4 * q4 + j] * inv_den);
      }
      *(uint2 *)(a.dob + row * D + d0) = pack_bf16x4(dv4[0], dv4[1], dv4[2], dv4[3]);
    }
  }
  const float dn = dn_p + shfl_xor32(dn_p);
  const float dg = dg_p + shfl_xor32(dg_p);
  const float gv = GATE ? 1.0f / (1.0f + __expf(-y)) : 1.0f;
  const float dy = GATE ? dg * gv * (1.0f - gv) : 0.0f;
  const float sc = gv * inv_den, dden = -gv * dg * inv_den;
  // da = S dnum + z dden (rows r).  The two terms largely cancel, so S and
  // dnum enter as bf16 pairs hi + lo (three products: hi hi, hi lo, lo hi)
  const uint16_t *sdb = a.comp ? a.sdc + qi * 32 * D : a.sd + (int64_t)bh * 32 * D;
  const uint16_t *sdl = sdb + (a.comp ? a.bh_count * a.nb : a.bh_count) * 32 * D;
  f32x16 da = f32x16{};
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 bh_, bl_;
#pragma unroll
      for (int e = 0; e < 8; ++e) split_bf16(dov[dt][8 * s2 + e] * sc, bh_, bl_, e);
      const int off = col * D + 32 * dt + 16 * s2 + 8 * g;
      const bf16x8 ah = *(const bf16x8 *)(sdb + off), al = *(const bf16x8 *)(sdl + off);
      da = mfma_bf16(ah, bh_, da);
      da = mfma_bf16(ah, bl_, da);
      da = mfma_bf16(al, bh_, da);
    }
  }
  float du[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + 4 * g + (i & 3);
    const float dai = da[i] + zr[i >> 2][i & 3] * dden;
    du[i] = (r < a.rank && valid) ? dai * (uacc[i] > 0.0f ? 1.0f : __expf(uacc[i])) : 0.0f;
  }
  bf16x8 duop[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) duop[i >> 3][i & 7] = (__bf16)du[i];
  // dRq = Wq du (rows d), then R^T and the gate term
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    f32x16 dr = f32x16{};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      dr = mfma_bf16(*(const bf16x8 *)(a.wqP + (32 * dt + col) * 32 + 16 * s2 + 8 * g), duop[s2], dr);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      float v4[4] = {dr[4 * q4], dr[4 * q4 + 1], dr[4 * q4 + 2], dr[4 * q4 + 3]};
      rope_back(v4[0], v4[1], d0, pt, ph, pw, sfreq[d0 / 2], a.rope);
      rope_back(v4[2], v4[3], d0 + 2, pt, ph, pw, sfreq[d0 / 2 + 1], a.rope);
      if (GATE) {
        const f32x4 w4 = *(const f32x4 *)(a.gate + d0);
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] += dy * w4[j];
      }
      f32x4 o = {v4[0], v4[1], v4[2], v4[3]};
      if (!valid) o = f32x4{0.f, 0.f, 0.f, 0.f};
      *(f32x4 *)(a.dqp + row * D + d0) = o;
    }
  }
  // per-token work arrays
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int r0 = 8 * q4 + 4 * g;
    const float s = valid ? sc : 0.0f;
    *(uint2 *)(a.ahat + row * 32 + r0) =
        pack_bf16x4(av[4 * q4] * s, av[4 * q4 + 1] * s, av[4 * q4 + 2] * s, av[4 * q4 + 3] * s);
    *(uint2 *)(a.duq + row * 32 + r0) = pack_bf16x4(du[4 * q4], du[4 * q4 + 1], du[4 * q4 + 2], du[4 * q4 + 3]);
  }
  if (lane < 32) {
    a.dn[row] = valid ? dn : 0.0f;
    a.dg[row] = valid ? dg : 0.0f;
    a.dy[row] = valid ? dy : 0.0f;
  }
}

// ----------------------------------------------------------- k_bwd_outer
// C[D][32] += sum over tokens of X[t][d] Y[t][r] on MFMA.  Each wave stages
// one 32-token tile of X (row-major, V-style swizzle) and of Y ([32][32]) in
// its own LDS area and reads both with the transposing LDS load, so the
// token index is the MFMA k index on both sides in the same order.
//   kOuterRopeQ: X = R(q), Y = dL/du (query)    -> dWq (summed over heads)
//   kOuterDout:  X = dO,   Y = g a / den        -> dS^T per head
//   kOuterRopeK: X = R(k), Y = dL/dw' (key)     -> dWk (summed over heads)
//   kOuterGate:  X = q,    Y = (dy, 0, ..., 0)  -> gate weights (column 0)
//   kOuterDoutBlk: as kOuterDout, one sum per query block (complement scope)
// Workgroup (p, bh) takes tiles p*4 + wave, p*4 + wave + 4*PP, ... of head bh
// and writes one fp32 partial [D][32] per wave; in kOuterDoutBlk it takes
// query blocks p*4 + wave, ... and writes each block's sum in bf16.
template <int D, int MODE>
__global__ __launch_bounds__(256) void k_bwd_outer(BwdArgs a, int PP) {
  constexpr int NS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(1024))) uint16_t sx[4][32 * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sy[4][32 * 32];
  __shared__ __attribute__((aligned(16))) float sfreq[D / 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, col = lane & 31;
  for (int p2 = tid; p2 < D / 2; p2 += 256) sfreq[p2] = rope_freq(2 * p2, a.rope);
  __syncthreads();
  const int bh = blockIdx.y, p = blockIdx.x;
  const int b = bh / a.heads, h = bh % a.heads;
  const int64_t base = (int64_t)b * a.stride_b + (int64_t)h * a.stride_h;
  const int64_t n_pad = (int64_t)a.nb * 64;
  uint16_t *X = sx[wave], *Y = sy[wave];
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  auto do_tile = [&](int tile) __attribute__((always_inline)) {
    const int64_t n = (int64_t)tile * 32 + col;
    const bool valid = n < a.n_tokens;
    const int64_t nc = valid ? n : a.n_tokens - 1;
    const int64_t row = (int64_t)bh * n_pad + n;
    // X row (8 dims per 16-byte chunk 2s + g), zero on padded tokens
    bf16x8 xr[NS];
    if (MODE == kOuterDout || MODE == kOuterDoutBlk) {
#pragma unroll
      for (int s = 0; s < NS; ++s) xr[s] = *(const bf16x8 *)(a.dob + row * D + 16 * s + 8 * g);
    } else {
      const uint16_t *src = (MODE == kOuterRopeK ? a.k : a.q) + base + nc * a.stride_n;
#pragma unroll
      for (int s = 0; s < NS; ++s) xr[s] = *(const bf16x8 *)(src + 16 * s + 8 * g);
      if (MODE == kOuterRopeQ || MODE == kOuterRopeK) {
        int pt, ph, pw;
        token_pos(nc, a.rope, pt, ph, pw);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f32x4 fr = *(const f32x4 *)&sfreq[8 * s + 4 * g];
          const float freq[4] = {fr[0], fr[1], fr[2], fr[3]};
          xr[s] = rope8(xr[s], 16 * s + 8 * g, pt, ph, pw, freq, a.rope);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = 2 * s + g;
      const u32x4 v = valid ? as_u32x4(xr[s]) : u32x4{0u, 0u, 0u, 0u};
      *(u32x4 *)(X + col * D + ((c ^ swz_v<D>(col)) << 3)) = v;
    }
    // Y row: 32 bf16 in 4 chunks, chunks 2g and 2g+1 from this lane
    u32x4 y0, y1;
    if (MODE == kOuterGate) {
      const float dyv = a.dy[row];
      y0 = u32x4{g == 0 ? (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)dyv) : 0u, 0u, 0u, 0u};
      y1 = u32x4{0u, 0u, 0u, 0u};
    } else {
      const uint16_t *ysrc = (MODE == kOuterRopeQ ? a.duq : (MODE == kOuterDout || MODE == kOuterDoutBlk) ? a.ahat : a.dwk_tok) + row * 32;
      y0 = *(const u32x4 *)(ysrc + 16 * g);
      y1 = *(const u32x4 *)(ysrc + 16 * g + 8);
    }
    *(u32x4 *)(Y + col * 32 + 16 * g) = y0;
    *(u32x4 *)(Y + col * 32 + 16 * g + 8) = y1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's tiles written
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 yb = vt_operand<32>(Y, s2, 0, lane);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma_bf16(vt_operand<D>(X, s2, dt, lane), yb, acc[dt]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next tile's writes
    };
  if constexpr (MODE == kOuterDoutBlk) {
    // one query block (two tiles) at a time: its dS_i^T in bf16
    for (int qb = p * 4 + wave; qb < a.nb; qb += 4 * PP) {
      do_tile(2 * qb);
      do_tile(2 * qb + 1);
      uint16_t *ob = a.pblk + ((int64_t)bh * a.nb + qb) * (D * 32);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = 32 * dt + 8 * (i >> 2) + 4 * g + (i & 3);
          ob[d * 32 + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[dt][i]);
        }
        acc[dt] = f32x16{};
      }
    }
    return;
  }
  for (int tile = p * 4 + wave; tile < 2 * a.nb; tile += 4 * PP) do_tile(tile);
  float *out = a.part + (((int64_t)bh * PP + p) * 4 + wave) * (D * 32);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 32 * dt + 8 * (i >> 2) + 4 * g + (i & 3);
      out[d * 32 + col] = acc[dt][i];
    }
  }
}

// ------------------------------------------------------------- k_bwd_sum
// Fixed-order sums of k_bwd_outer's partials, per head over its 4*PP
// partials, into dst [BH][D*32] (dS^T, or the per-head parts of the pooled
// gradients).
template <int D>
__global__ __launch_bounds__(256) void k_bwd_sum(BwdArgs a, int PP, float *dst) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= D * 32) return;
  const int bh = blockIdx.y;
  const int64_t np = 4LL * PP;
  const float *p = a.part + (int64_t)bh * np * (D * 32) + idx;
  float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t c = 0;
  for (; c + 8 <= np; c += 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc8[i] += p[(c + i) * (D * 32)];
  }
  for (int i = 0; c + i < np; ++i) acc8[i] += p[(c + i) * (D * 32)];
  dst[(int64_t)bh * D * 32 + idx] =
      ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
}

// The pooled gradients: the per-head sums of k_bwd_sum added over heads in
// order, written as [D][rank] (dWq, dWk) or, for the gate, column 0 as
// dgate[0..D) plus the per-head bias sums (at part[bias_at ...]) as dgate[D].
template <int D, bool GATE>
__global__ __launch_bounds__(256) void k_bwd_sum_heads(BwdArgs a, const float *heads, int64_t bias_at,
                                                       float *dst) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= D * 32) return;
  float acc = 0.0f;
  for (int64_t h = 0; h < a.bh_count; ++h) acc += heads[h * D * 32 + idx];
  const int d = idx / 32, r = idx % 32;
  if (GATE) {
    if (r == 0) dst[d] = acc;
    if (idx == 0) {
      float bsum = 0.0f;
      for (int64_t i = 0; i < a.bh_count; ++i) bsum += a.part[bias_at + i];
      dst[D] = bsum;
    }
  } else if (r < a.rank) {
    dst[d * a.rank + r] = acc;
  }
}

// -------------------------------------------------------------- k_bwd_dz
// Per head: dz[r] = sum_t dden_t a_t[r] = -sum_t dg_t (g a / den)_t[r] and
// the gate-bias partial sum_t dy_t.  First level: workgroup (p, bh) sums the
// tokens p*per .. (p+1)*per into part[(bh*PZ + p)*33 + (r | 32)]; second
// level (k_bwd_dz2): per head over p in order, into dz and part[bias_at + bh].
constexpr int kDzParts = 64;
__global__ __launch_bounds__(256) void k_bwd_dz(BwdArgs a) {
  __shared__ float red[8][33];
  const int tid = threadIdx.x, r = tid & 31, lane8 = tid >> 5;
  const int p = blockIdx.x, bh = blockIdx.y;
  const int64_t n_pad = (int64_t)a.nb * 64, row0 = (int64_t)bh * n_pad;
  const int64_t per = (a.n_tokens + kDzParts - 1) / kDzParts;
  const int64_t n0 = p * per, n1 = min<int64_t>(a.n_tokens, n0 + per);
  float acc = 0.0f, yb = 0.0f;
  for (int64_t n = n0 + lane8; n < n1; n += 8) {
    acc -= a.dg[row0 + n] * __builtin_bit_cast(float, ((uint32_t)a.ahat[(row0 + n) * 32 + r]) << 16);
    if (r == 0) yb += a.dy[row0 + n];
  }
  red[lane8][r] = acc;
  if (r == 0) red[lane8][32] = yb;
  __syncthreads();
  if (tid < 33) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += red[i][tid];
    a.part[((int64_t)bh * kDzParts + p) * 33 + tid] = s;
  }
}

__global__ __launch_bounds__(64) void k_bwd_dz2(BwdArgs a, int64_t bias_at) {
  const int tid = threadIdx.x, bh = blockIdx.x;
  if (tid >= 33) return;
  float s = 0.0f;
  for (int p = 0; p < kDzParts; ++p) s += a.part[((int64_t)bh * kDzParts + p) * 33 + tid];
  if (tid < 32) a.dz[(int64_t)bh * 32 + tid] = tid < a.rank ? s : 0.0f;
  else a.part[bias_at + bh] = s;
}

// ----------------------------------------------------------- k_bwd_dsops
// dS as bf16 operands: dsr [32][D] (rows r, natural d) and dst [D][32]
// (rows d, rank permuted).
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dsops(BwdArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.bh_count * D * 32) return;
  const int64_t bh = t / (D * 32);
  const int e = (int)(t % (D * 32)), d = e / 32, r = e % 32;
  const __bf16 v = (__bf16)a.ds32[t];
  a.dsr[bh * 32 * D + r * D + d] = __builtin_bit_cast(uint16_t, v);
  a.dst[bh * D * 32 + d * 32 + perm16_key_of_pos(r)] = __builtin_bit_cast(uint16_t, v);
}

// ------------------------------------------------------ complement scope
// Query block i's low-rank term reads S_i = sum of the states S_j of the key
// blocks i does not keep, so the gradient of a block state is
//   dS_j = sum over query blocks i that do not keep j of dS_i
//        = (sum over all i of dS_i) - sum over the i that keep j of dS_i,
// with dS_i = sum over i's tokens of (g a / den) dO^T, and dz_j likewise
// from dz_i = -sum over i's tokens of dg (g a / den).  The per-query-block
// sums are bf16 (dS_i) and fp32 (dz_i); the head totals add the same bf16
// values in fp32, in block order.

// dz_i: one wave per query block, lane (half, r) summing 32 tokens for rank r
__global__ __launch_bounds__(256) void k_bwd_dzblk(BwdArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 31, hf = lane >> 5;
  const int bh = blockIdx.y, qb = blockIdx.x * 4 + wave;
  if (qb >= a.nb) return;
  const int64_t n_pad = (int64_t)a.nb * 64;
  const int64_t row0 = (int64_t)bh * n_pad + (int64_t)qb * 64 + 32 * hf;
  float acc = 0.0f;
  for (int t = 0; t < 32; ++t)
    acc -= a.dg[row0 + t] * __builtin_bit_cast(float, ((uint32_t)a.ahat[(row0 + t) * 32 + r]) << 16);
  acc += __shfl_xor(acc, 32, 64);
  if (hf == 0) a.dzblk[((int64_t)bh * a.nb + qb) * 32 + r] = acc;
}

// head totals of dS_i^T into ds32 [BH][D*32], in block order
template <int D>
__global__ __launch_bounds__(256) void k_bwd_sumblk(BwdArgs a) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= D * 32) return;
  const int bh = blockIdx.y;
  const uint16_t *p = a.pblk + (int64_t)bh * a.nb * (D * 32) + idx;
  float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto at = [&](int64_t i) { return __builtin_bit_cast(float, ((uint32_t)p[i * (D * 32)]) << 16); };
  int64_t i = 0;
  for (; i + 8 <= a.nb; i += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc8[u] += at(i + u);
  }
  for (int u = 0; i + u < a.nb; ++u) acc8[u] += at(i + u);
  a.ds32[(int64_t)bh * D * 32 + idx] =
      ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
}

// dS_j, dz_j per key block j: the head total minus the sums of the query
// blocks that keep j (the transposed map), written as the bf16 operand copies
// of k_bwd_key (dsrc as dsr, dstc as dst) and dz_j in fp32.  One workgroup per
// key block; thread t owns elements [t*D/8, (t+1)*D/8) of the [D][32] sum.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dsc(BwdArgs a) {
  constexpr int EPT = D / 8;
  typedef const __attribute__((address_space(4))) int32_t *cint_p;
  const int tid = threadIdx.x, j = blockIdx.x, bh = blockIdx.y;
  const int64_t kj = (int64_t)bh * a.nb + j;
  const int cnt = ((cint_p)a.tcount)[kj];
  const cint_p list = (cint_p)(a.tlist + kj * a.nb);
  const uint16_t *pb = a.pblk + (int64_t)bh * a.nb * (D * 32) + tid * EPT;
  const float *zb = a.dzblk + (int64_t)bh * a.nb * 32 + 4 * tid;
  float acc[EPT], az[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.0f;
  for (int t = 0; t < cnt; ++t) {
    const int64_t i = list[t];
    const u32x4 *src = (const u32x4 *)(pb + i * (D * 32));
#pragma unroll
    for (int c = 0; c < EPT / 8; ++c) {
      const u32x4 w = src[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[8 * c + 2 * e] += bflo(w[e]);
        acc[8 * c + 2 * e + 1] += bfhi(w[e]);
      }
    }
    if (tid < 8) {
      const f32x4 zz = *(const f32x4 *)(zb + i * 32);
#pragma unroll
      for (int e = 0; e < 4; ++e) az[e] += zz[e];
    }
  }
  const float *tot = a.ds32 + (int64_t)bh * D * 32 + tid * EPT;
  uint16_t *dr = a.dsrc + kj * 32 * D, *dt = a.dstc + kj * D * 32;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int idx = tid * EPT + e, d = idx / 32, r = idx % 32;
    const uint16_t v = __builtin_bit_cast(uint16_t, (__bf16)(tot[e] - acc[e]));
    dr[r * D + d] = v;
    dt[d * 32 + perm16_key_of_pos(r)] = v;
  }
  if (tid < 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * tid + e;
      a.dzc[kj * 32 + r] = r < a.rank ? a.dz[(int64_t)bh * 32 + r] - az[e] : 0.0f;
    }
  }
}

// ------------------------------------------------------------- k_bwd_key
// One wave per 32-token tile of keys: b = phi(Wk^T R(k)), db = dS v + dz,
// dw' = db phi'(.), the low-rank parts of dk (R^T(Wk dw')) and dv (dS^T b).
template <int D>
__global__ __launch_bounds__(256) void k_bwd_key(BwdArgs a) {
  constexpr int NS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) float sfreq[D / 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, col = lane & 31;
  for (int p2 = tid; p2 < D / 2; p2 += 256) sfreq[p2] = rope_freq(2 * p2, a.rope);
  __syncthreads();
  const int bh = blockIdx.y;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= 2 * a.nb) return;
  const int b = bh / a.heads, h = bh % a.heads;
  const int64_t base = (int64_t)b * a.stride_b + (int64_t)h * a.stride_h;
  const int64_t n_pad = (int64_t)a.nb * 64;
  const int64_t m = (int64_t)tile * 32 + col;
  const bool valid = m < a.n_tokens;
  const int64_t mc = valid ? m : a.n_tokens - 1;
  const int64_t row = (int64_t)bh * n_pad + m;
  bf16x8 kreg[NS], vreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kreg[s] = *(const bf16x8 *)(a.k + base + mc * a.stride_n + 16 * s + 8 * g);
    vreg[s] = *(const bf16x8 *)(a.v + base + mc * a.stride_n + 16 * s + 8 * g);
  }
  int pt, ph, pw;
  token_pos(mc, a.rope, pt, ph, pw);
  f32x16 wacc = f32x16{}, db = f32x16{};
  // dS and dz of the head, or (complement scope) of this key block
  const int64_t kj = (int64_t)bh * a.nb + (tile >> 1);
  const uint16_t *dsb = a.comp ? a.dsrc + kj * 32 * D : a.dsr + (int64_t)bh * 32 * D;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const f32x4 fr = *(const f32x4 *)&sfreq[8 * s + 4 * g];
    const float freq[4] = {fr[0], fr[1], fr[2], fr[3]};
    const bf16x8 kr = rope8(kreg[s], 16 * s + 8 * g, pt, ph, pw, freq, a.rope);
    wacc = mfma_bf16(*(const bf16x8 *)(a.wkT + col * D + 16 * s + 8 * g), kr, wacc);
    db = mfma_bf16(*(const bf16x8 *)(dsb + col * D + 16 * s + 8 * g), vreg[s], db);
  }
  const f32x4 *dzb = (const f32x4 *)(a.comp ? a.dzc + kj * 32 : a.dz + (int64_t)bh * 32);
  float bv[16], dw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + 4 * g + (i & 3);
    const bool ok = r < a.rank && valid;
    const float dzr = dzb[2 * (i >> 2) + g][i & 3];
    bv[i] = ok ? phi(wacc[i]) : 0.0f;
    dw[i] = ok ? (db[i] + dzr) * (wacc[i] > 0.0f ? 1.0f : __expf(wacc[i])) : 0.0f;
  }
  bf16x8 bop[2], dwop[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    bop[i >> 3][i & 7] = (__bf16)bv[i];
    dwop[i >> 3][i & 7] = (__bf16)dw[i];
  }
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    *(uint2 *)(a.dwk_tok + row * 32 + 8 * q4 + 4 * g) =
        pack_bf16x4(dw[4 * q4], dw[4 * q4 + 1], dw[4 * q4 + 2], dw[4 * q4 + 3]);
  const uint16_t *dstb = a.comp ? a.dstc + kj * D * 32 : a.dst + (int64_t)bh * D * 32;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    f32x16 dv = f32x16{}, dr = f32x16{};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      dv = mfma_bf16(*(const bf16x8 *)(dstb + (32 * dt + col) * 32 + 16 * s2 + 8 * g), bop[s2], dv);
      dr = mfma_bf16(*(const bf16x8 *)(a.wkP + (32 * dt + col) * 32 + 16 * s2 + 8 * g), dwop[s2], dr);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      float k4[4] = {dr[4 * q4], dr[4 * q4 + 1], dr[4 * q4 + 2], dr[4 * q4 + 3]};
      rope_back(k4[0], k4[1], d0, pt, ph, pw, sfreq[d0 / 2], a.rope);
      rope_back(k4[2], k4[3], d0 + 2, pt, ph, pw, sfreq[d0 / 2 + 1], a.rope);
      f32x4 ok = {k4[0], k4[1], k4[2], k4[3]};
      f32x4 ov = {dv[4 * q4], dv[4 * q4 + 1], dv[4 * q4 + 2], dv[4 * q4 + 3]};
      if (!valid) ok = ov = f32x4{0.f, 0.f, 0.f, 0.f};
      *(f32x4 *)(a.dkp + row * D + d0) = ok;
      *(f32x4 *)(a.dvp + row * D + d0) = ov;
    }
  }
}

// ------------------------------------------------------------- tile copies
// Copy 64 token rows of a bf16 matrix (row stride `stride` elements, rows
// past `last` taken from row `last`) into an LDS tile, row-major with the
// V-style chunk swizzle, 16 bytes per lane per op; `ops` ops per thread of a
// 128-thread workgroup, thread tid taking chunks o*128 + tid.
template <int D>
static __device__ __forceinline__ void copy_tile64(const uint16_t *src, int64_t stride, int64_t r0,
                                                   int64_t last, uint16_t *tile, int tid) {
  constexpr int CH = D / 8, OPS = 64 * CH / 128;
  const int wave = tid >> 6;
#pragma unroll
  for (int o = 0; o < OPS; ++o) {
    const int cidx = o * 128 + tid;
    const int row = cidx / CH, pc = cidx % CH;
    const int64_t sr = min(r0 + row, last);
    lds_dma16(src + sr * stride + ((pc ^ swz_v<D>(row)) << 3), tile + (o * 128 + wave * 64) * 8);
  }
}

// 16-byte MFMA operand from row `row` of a V-style swizzled tile: dims
// 16 s + 8 g .. +8 (logical chunk 2 s + g)
template <int D>
static __device__ __forceinline__ bf16x8 row_operand(const uint16_t *tile, int row, int s, int g) {
  return *(const bf16x8 *)(tile + row * D + (((2 * s + g) ^ swz_v<D>(row)) << 3));
}

// -------------------------------------------------------------- k_bwd_dq
// One workgroup (2 waves, 32 queries each) per query block, with K and V
// tiles of its kept key blocks in a two-slot LDS ring: S^T = K Q^T and
// dP^T = V dO^T as in the forward's transposed form, dS^T = P^T (dP^T - D),
// dq^T += K^T dS^T on MFMA.  dS enters as a bf16 pair hi + lo (about 16
// significant bits): its terms cancel in the sum over keys.  Adds the
// low-rank part and writes dq in bf16.
template <int D>
__global__ __launch_bounds__(128) void k_bwd_dq(BwdArgs a) {
  constexpr int NS = D / 16, DT = D / 32, TILE = 64 * D, OPS = 2 * (64 * (D / 8)) / 128;
  __shared__ __attribute__((aligned(1024))) uint16_t ring[2][2 * TILE];
  const int tid = threadIdx.x, lane = tid & 63, half = tid >> 6, g = lane >> 5, col = lane & 31;
  const int qb = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.heads, h = bh % a.heads;
  const int64_t base = (int64_t)b * a.stride_b + (int64_t)h * a.stride_h;
  const int64_t n_pad = (int64_t)a.nb * 64;
  const int64_t n = (int64_t)qb * 64 + 32 * half + col;
  const bool valid = n < a.n_tokens;
  const int64_t nc = valid ? n : a.n_tokens - 1;
  const int64_t row = (int64_t)bh * n_pad + n;
  bf16x8 qreg[NS], doreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qreg[s] = *(const bf16x8 *)(a.q + base + nc * a.stride_n + 16 * s + 8 * g);
    doreg[s] = *(const bf16x8 *)(a.dob + row * D + 16 * s + 8 * g);
  }
  const float lse2 = valid ? a.lse[row] : 0.0f;
  const float dn = a.dn[row];
  // the block map through the scalar cache (uniform per workgroup)
  typedef const __attribute__((address_space(4))) int32_t *cint_p;
  const cint_p mrow = (cint_p)(a.map + ((int64_t)bh * a.nb + qb) * a.kb);
  const int kb = a.kb;
  wait_vmcnt<0>();
  auto issue = [&](int t, int slot) __attribute__((always_inline)) {
    const int j = __builtin_amdgcn_readfirstlane(mrow[t]);
    copy_tile64<D>(a.k + base, a.stride_n, (int64_t)j * 64, a.n_tokens - 1, ring[slot], tid);
    copy_tile64<D>(a.v + base, a.stride_n, (int64_t)j * 64, a.n_tokens - 1, ring[slot] + TILE, tid);
  };
  issue(0, 0);
  if (kb > 1) issue(1, 1);
  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};
  const float c = a.scale_log2e;
  for (int t = 0; t < kb; ++t) {
    if (t + 1 < kb) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
    __syncthreads();
    const uint16_t *sK = ring[t & 1], *sV = ring[t & 1] + TILE;
    const int j = __builtin_amdgcn_readfirstlane(mrow[t]);
    const int lim = (int)min<int64_t>(64, a.n_tokens - (int64_t)j * 64);  // valid keys of the block
    bf16x8 dshi[4], dslo[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sacc = mfma_bf16(row_operand<D>(sK, 32 * h2 + col, s, g), qreg[s], sacc);
        dpacc = mfma_bf16(row_operand<D>(sV, 32 * h2 + col, s, g), doreg[s], dpacc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * h2 + 8 * (i >> 2) + 4 * g + (i & 3);
        const float pv = (valid && key < lim) ? fast_exp2(__builtin_fmaf(sacc[i], c, -lse2)) : 0.0f;
        split_bf16(pv * (dpacc[i] - dn), dshi[2 * h2 + (i >> 3)], dslo[2 * h2 + (i >> 3)], i & 7);
      }
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 kt = vt_operand<D>(sK, s4, dt, lane);
        dq[dt] = mfma_bf16(kt, dshi[s4], dq[dt]);
        dq[dt] = mfma_bf16(kt, dslo[s4], dq[dt]);
      }
    __syncthreads();
    if (t + 2 < kb) issue(t + 2, t & 1);
  }
  uint16_t *orow = a.dq + base + n * a.stride_n;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      const f32x4 lr = *(const f32x4 *)(a.dqp + row * D + d0);
      float v[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) v[jj] = valid ? a.scale * dq[dt][4 * q4 + jj] + lr[jj] : 0.0f;
      *(uint2 *)(orow + d0) = pack_bf16x4(v[0], v[1], v[2], v[3]);
    }
  }
}

// ------------------------------------------------------------- k_bwd_dqg
// Sparse dq on the forward's group schedule (k_order, k_group, k_union of the
// recompute): one workgroup per group of G query blocks, waves 2m and 2m+1
// owning rows 0-31 and 32-63 of member m, walks the group's union list two
// tiles per barrier through a four-slot ring of K and V tiles, as k_attn
// does, so that each key block is copied once for every member that kept it
// and two waves share each SIMD.  Per listed block and 32-key half, a member
// wave forms S^T = K Q^T and dP^T = V dO^T (K and V rows), dS^T = P^T
// (dP^T - D) as a bf16 pair hi + lo, and dq^T += K^T dS^T (K read
// transposed).  Unions that can be longer than the LDS copy (kDqgLmax
// entries) take k_bwd_dq.
constexpr int kDqgLmax = 2048;

template <int D, int G>
__global__ __launch_bounds__(128 * G, 2) void k_bwd_dqg(BwdArgs a) {
  constexpr int NS = D / 16, DT = D / 32, TILE = 64 * D, CH = D / 8;
  constexpr int NT = 128 * G;
  constexpr int OPS = (64 * CH) / NT;  // copies per thread per tensor per tile
  static_assert(OPS >= 1 && (64 * CH) % NT == 0, "tile split");
  constexpr int S = 4;
  __shared__ __attribute__((aligned(1024))) uint16_t ring[S * 2 * TILE];
  __shared__ int32_t slist[kDqgLmax + 8];  // + room for the reads ahead past the end
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, col = lane & 31;
  const int member = wave >> 1, half = wave & 1;
  const int64_t L = blockIdx.x;
  const int64_t sidx = L / 8;
  const int64_t bh64 = sidx / a.groups_per_xcd;
  const int64_t group = (L % 8) * a.groups_per_xcd + sidx % a.groups_per_xcd;
  if (bh64 >= a.bh_count || group >= a.ngroups) return;
  const int bh = (int)bh64;
  const int64_t gidx = (int64_t)bh * a.ngroups + group;
  typedef const __attribute__((address_space(4))) int32_t *cint_p;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qb = ((cint_p)a.ugroup)[gidx * G + (wave_u >> 1)];
  const bool active = qb >= 0;
  const int b = bh / a.heads, h = bh % a.heads;
  const int64_t base = (int64_t)b * a.stride_b + (int64_t)h * a.stride_h;
  const int64_t n_pad = (int64_t)a.nb * 64;
  const int64_t n = (int64_t)(active ? qb : 0) * 64 + 32 * half + col;
  const bool valid = active && n < a.n_tokens;
  const int64_t nc = n < a.n_tokens ? n : a.n_tokens - 1;
  const int64_t row = (int64_t)bh * n_pad + n;
  const int32_t *list = a.ulist + gidx * a.list_stride;
  const int U = ((cint_p)a.ucount)[gidx];
  const uint16_t *Kb = a.k + base, *Vb = a.v + base;
  // this thread's byte offsets inside a key block (V-style swizzle, the
  // layout row_operand and vt_operand read)
  uint32_t goff[OPS];
#pragma unroll
  for (int o = 0; o < OPS; ++o) {
    const int cidx = o * NT + tid;
    const int r = cidx / CH, pc = cidx % CH;
    goff[o] = (uint32_t)(((int64_t)r * a.stride_n + ((pc ^ swz_v<D>(r)) * 8)) * 2);
  }
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  auto issue_j = [&](int t, int j) __attribute__((always_inline)) {
    uint16_t *slot = ring + (t % S) * (2 * TILE);
    const int64_t jrow = (int64_t)j * 64;
    if (jrow + 64 <= a.n_tokens) {
      const uint16_t *kj = Kb + jrow * a.stride_n, *vj = Vb + jrow * a.stride_n;
      const uint32_t m0 = ring_lds + (uint32_t)((t % S) * (2 * TILE) * 2) + (uint32_t)wave_u * 1024u;
#pragma unroll
      for (int o = 0; o < OPS; ++o) {
        lds_dma16_m0(kj, goff[o], m0 + (uint32_t)(o * NT * 16));
        lds_dma16_m0(vj, goff[o], m0 + (uint32_t)(TILE * 2 + o * NT * 16));
      }
    } else {
#pragma unroll
      for (int o = 0; o < OPS; ++o) {
        const int cidx = o * NT + tid;
        const int r = cidx / CH, pc = cidx % CH;
        // rows past N (tail block) are copied from row N-1: finite values,
        // masked out of P
        const int64_t src = min(jrow + r, a.n_tokens - 1) * a.stride_n + ((pc ^ swz_v<D>(r)) * 8);
        lds_dma16(Kb + src, slot + (o * NT + wave * 64) * 8);
        lds_dma16(Vb + src, slot + TILE + (o * NT + wave * 64) * 8);
      }
    }
  };
  // prologue: tiles 0 and 1, this wave's Q and dO rows and the list in flight together
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (t < U) issue_j(t, ((cint_p)list)[t] & 0xffff);
  bf16x8 qreg[NS], doreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qreg[s] = *(const bf16x8 *)(a.q + base + nc * a.stride_n + 16 * s + 8 * g);
    doreg[s] = *(const bf16x8 *)(a.dob + row * D + 16 * s + 8 * g);
  }
  const float lse2 = valid ? a.lse[row] : 0.0f;
  const float dn = a.dn[row];
  {
    int32_t lv[(kDqgLmax + NT - 1) / NT];
#pragma unroll
    for (int r = 0; r < (kDqgLmax + NT - 1) / NT; ++r) {
      const int i = r * NT + tid;
      lv[r] = i < U ? list[i] : 0;
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int r = 0; r < (kDqgLmax + NT - 1) / NT; ++r) {
      const int i = r * NT + tid;
      if (i < U) slist[i] = lv[r];
    }
  }
  __syncthreads();  // tiles 0 and 1 and the list complete for every wave
  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};
  const float c = a.scale_log2e;
  auto tile = [&](int t, int ent) __attribute__((always_inline)) {
    const int j = ent & 0xffff;
    const uint16_t *sK = ring + (t % S) * (2 * TILE), *sV = sK + TILE;
    const int lim = (int)min<int64_t>(64, a.n_tokens - (int64_t)j * 64);  // valid keys of the block
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sacc = mfma_bf16(row_operand<D>(sK, 32 * h2 + col, s, g), qreg[s], sacc);
        dpacc = mfma_bf16(row_operand<D>(sV, 32 * h2 + col, s, g), doreg[s], dpacc);
      }
      bf16x8 dshi[2], dslo[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * h2 + 8 * (i >> 2) + 4 * g + (i & 3);
        const float pv = (valid && key < lim) ? fast_exp2(__builtin_fmaf(sacc[i], c, -lse2)) : 0.0f;
        split_bf16(pv * (dpacc[i] - dn), dshi[i >> 3], dslo[i >> 3], i & 7);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 kt = vt_operand<D>(sK, 2 * h2 + s2, dt, lane);
          dq[dt] = mfma_bf16(kt, dshi[s2], dq[dt]);
          dq[dt] = mfma_bf16(kt, dslo[s2], dq[dt]);
        }
    }
  };
  // two tiles per barrier: iteration k consumes tiles 2k and 2k+1 and first
  // copies 2k+2 and 2k+3 into the slots of 2k-2 and 2k-1 (free once every
  // wave has passed the barrier); list entries are read one iteration ahead
  int ea = slist[0], eb = slist[1], ec = slist[2], ed = slist[3];
  for (int t2 = 0; t2 < U; t2 += 2) {
    wait_vmcnt<0>();  // this wave's copies of tiles t2, t2+1
    barrier_lds();    // both visible to all waves; every wave is done with t2-2, t2-1
    const int e0 = ea, e1 = eb;
    if (t2 + 2 < U) issue_j(t2 + 2, __builtin_amdgcn_readfirstlane(ec & 0xffff));
    if (t2 + 3 < U) issue_j(t2 + 3, __builtin_amdgcn_readfirstlane(ed & 0xffff));
    ea = ec;
    eb = ed;
    ec = slist[t2 + 4];
    ed = slist[t2 + 5];
    const bool m0 = active && ((e0 >> (16 + member)) & 1);
    const bool m1 = active && t2 + 1 < U && ((e1 >> (16 + member)) & 1);
    if (m0) tile(t2, e0);
    if (m1) tile(t2 + 1, e1);
  }
  if (!active) return;
  uint16_t *orow = a.dq + base + n * a.stride_n;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      const f32x4 lr = *(const f32x4 *)(a.dqp + row * D + d0);
      float v[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) v[jj] = valid ? a.scale * dq[dt][4 * q4 + jj] + lr[jj] : 0.0f;
      *(uint2 *)(orow + d0) = pack_bf16x4(v[0], v[1], v[2], v[3]);
    }
  }
}

// ------------------------------------------------------------ k_bwd_tmap
// For each key block j of a head: the query blocks that kept it, ascending.
// k_bwd_mapbits turns each map row into a bitset over key blocks; k_bwd_tmap
// then scans, for its key block, bit j of every row in order (independent
// loads, shared by the 32 key blocks of a word).
__global__ __launch_bounds__(64) void k_bwd_mapbits(BwdArgs a) {
  extern __shared__ uint32_t bits[];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int W = (a.nb + 31) / 32;
  for (int w = tid; w < W; w += 64) bits[w] = 0u;
  __syncthreads();
  const int32_t *mr = a.map + ((int64_t)bh * a.nb + i) * a.kb;
  for (int t = tid; t < a.kb; t += 64) {
    const int j = mr[t];
    atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  uint32_t *out = (uint32_t *)a.tbits + ((int64_t)bh * a.nb + i) * W;
  for (int w = tid; w < W; w += 64) out[w] = bits[w];
}

__global__ __launch_bounds__(256) void k_bwd_tmap(BwdArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (j >= a.nb) return;
  const int W = (a.nb + 31) / 32;
  const uint32_t *col = (const uint32_t *)a.tbits + (int64_t)bh * a.nb * W + (j >> 5);
  const uint32_t bit = 1u << (j & 31);
  int32_t *out = a.tlist + ((int64_t)bh * a.nb + j) * a.nb;
  int cnt = 0;
  int i = 0;
  for (; i + 8 <= a.nb; i += 8) {
    uint32_t w8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w8[u] = col[(int64_t)(i + u) * W];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (w8[u] & bit) out[cnt++] = i + u;
  }
  for (; i < a.nb; ++i)
    if (col[(int64_t)i * W] & bit) out[cnt++] = i;
  a.tcount[(int64_t)bh * a.nb + j] = cnt;
}

// ------------------------------------------------------------- k_bwd_dkv
// One workgroup (2 waves, 32 keys each) per key block: walks the query blocks
// that kept it with Q, dO, their log-sum-exp and D rows in a two-slot LDS
// ring, and accumulates dv^T = dO^T P and dk^T = Q^T dS on MFMA, keys as the
// lane column (S = Q K^T, dP = dO V^T).  Adds the low-rank parts and writes
// dk, dv in bf16.
template <int D>
__global__ __launch_bounds__(128) void k_bwd_dkv(BwdArgs a) {
  constexpr int NS = D / 16, DT = D / 32, TILE = 64 * D, OPS = 2 * (64 * (D / 8)) / 128 + 1;
  constexpr int SLOT = 2 * TILE + 256;  // Q, dO, then 64 lse + 64 D floats
  __shared__ __attribute__((aligned(1024))) uint16_t ring[2][SLOT];
  const int tid = threadIdx.x, lane = tid & 63, half = tid >> 6, g = lane >> 5, col = lane & 31;
  const int kbk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.heads, h = bh % a.heads;
  const int64_t base = (int64_t)b * a.stride_b + (int64_t)h * a.stride_h;
  const int64_t n_pad = (int64_t)a.nb * 64;
  const int64_t m = (int64_t)kbk * 64 + 32 * half + col;
  const bool valid = m < a.n_tokens;
  const int64_t mc = valid ? m : a.n_tokens - 1;
  const int64_t row = (int64_t)bh * n_pad + m;
  bf16x8 kreg[NS], vreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kreg[s] = *(const bf16x8 *)(a.k + base + mc * a.stride_n + 16 * s + 8 * g);
    vreg[s] = *(const bf16x8 *)(a.v + base + mc * a.stride_n + 16 * s + 8 * g);
  }
  typedef const __attribute__((address_space(4))) int32_t *cint_p;
  const int cnt = ((cint_p)a.tcount)[(int64_t)bh * a.nb + kbk];
  const cint_p list = (cint_p)(a.tlist + ((int64_t)bh * a.nb + kbk) * a.nb);
  wait_vmcnt<0>();
  auto issue = [&](int t, int slot) __attribute__((always_inline)) {
    const int i = __builtin_amdgcn_readfirstlane(list[t]);
    copy_tile64<D>(a.q + base, a.stride_n, (int64_t)i * 64, a.n_tokens - 1, ring[slot], tid);
    copy_tile64<D>(a.dob + (int64_t)bh * n_pad * D, D, (int64_t)i * 64, n_pad - 1, ring[slot] + TILE, tid);
    // lse (wave 0) and D (wave 1) of the 64 rows: 16 lanes x 16 bytes each
    const float *src = (half == 0 ? a.lse : a.dn) + (int64_t)bh * n_pad + (int64_t)i * 64;
    uint16_t *dst = ring[slot] + 2 * TILE + half * 128;
    if (lane < 16) lds_dma16(src + 4 * lane, dst);
  };
  if (cnt > 0) issue(0, 0);
  if (cnt > 1) issue(1, 1);
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16{};
  const float c = a.scale_log2e;
  for (int t = 0; t < cnt; ++t) {
    if (t + 1 < cnt) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
    __syncthreads();
    const uint16_t *sQ = ring[t & 1], *sO = ring[t & 1] + TILE;
    const float *slse = (const float *)(ring[t & 1] + 2 * TILE), *sdn = slse + 64;
    const int i = __builtin_amdgcn_readfirstlane(list[t]);
    const int lim = (int)min<int64_t>(64, a.n_tokens - (int64_t)i * 64);  // valid query rows
    // P and dS in bf16: the sums over query rows here do not cancel the way
    // dS does over keys (k_bwd_dq), so one rounding suffices
    bf16x8 pop[4], dsop[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sacc = mfma_bf16(row_operand<D>(sQ, 32 * h2 + col, s, g), kreg[s], sacc);
        dpacc = mfma_bf16(row_operand<D>(sO, 32 * h2 + col, s, g), vreg[s], dpacc);
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r0 = 32 * h2 + 8 * q4 + 4 * g;
        const f32x4 l4 = *(const f32x4 *)(slse + r0);
        const f32x4 d4 = *(const f32x4 *)(sdn + r0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * q4 + j;
          const float pv = (r0 + j < lim) ? fast_exp2(__builtin_fmaf(sacc[e], c, -l4[j])) : 0.0f;
          pop[2 * h2 + (e >> 3)][e & 7] = (__bf16)pv;
          dsop[2 * h2 + (e >> 3)][e & 7] = (__bf16)(pv * (dpacc[e] - d4[j]));
        }
      }
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 ot = vt_operand<D>(sO, s4, dt, lane), qt = vt_operand<D>(sQ, s4, dt, lane);
        dv[dt] = mfma_bf16(ot, pop[s4], dv[dt]);
        dk[dt] = mfma_bf16(qt, dsop[s4], dk[dt]);
      }
    }
    __syncthreads();
    if (t + 2 < cnt) issue(t + 2, t & 1);
  }
  uint16_t *krow = a.dk + base + m * a.stride_n, *vrow = a.dv + base + m * a.stride_n;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      const f32x4 lk = *(const f32x4 *)(a.dkp + row * D + d0);
      const f32x4 lv = *(const f32x4 *)(a.dvp + row * D + d0);
      float vk[4], vv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vk[j] = valid ? a.scale * dk[dt][4 * q4 + j] + lk[j] : 0.0f;
        vv[j] = valid ? dv[dt][4 * q4 + j] + lv[j] : 0.0f;
      }
      *(uint2 *)(krow + d0) = pack_bf16x4(vk[0], vk[1], vk[2], vk[3]);
      *(uint2 *)(vrow + d0) = pack_bf16x4(vv[0], vv[1], vv[2], vv[3]);
    }
  }
}

// ------------------------------------------------------------- launchers
static int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

int bwd_outer_parts(int64_t bh_count, int nb, int mode) {
  // per head about 256 tiles per workgroup pass for the pooled modes; the
  // per-head dS reduction uses more workgroups per head
  (void)mode;
  const int tiles = 2 * nb;
  const int want = (int)std::max<int64_t>(1, 2048 / std::max<int64_t>(1, bh_count));
  return std::max(1, std::min(want, cdiv(tiles, 4)));
}

void launch_bwd_prep(const BwdArgs &a, int D, hipStream_t st) {
  const dim3 grid(cdiv(std::max<int64_t>(D * 32, a.bh_count * 32 * D), 256), 2);
  if (D == 64) hipLaunchKernelGGL(k_bwd_prep<64>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_prep<128>, grid, dim3(256), 0, st, a);
}

void launch_bwd_query(const BwdArgs &a, int D, hipStream_t st) {
  const dim3 grid(cdiv(2 * a.nb, 4), (unsigned)a.bh_count);
  const bool gate = a.gate != nullptr, f32 = a.dout_f32 != 0;
#define ROLA_BQ(DD, GG, FF) hipLaunchKernelGGL((k_bwd_query<DD, GG, FF>), grid, dim3(256), 0, st, a)
  if (D == 64) {
    if (gate) { if (f32) ROLA_BQ(64, true, true); else ROLA_BQ(64, true, false); }
    else { if (f32) ROLA_BQ(64, false, true); else ROLA_BQ(64, false, false); }
  } else {
    if (gate) { if (f32) ROLA_BQ(128, true, true); else ROLA_BQ(128, true, false); }
    else { if (f32) ROLA_BQ(128, false, true); else ROLA_BQ(128, false, false); }
  }
#undef ROLA_BQ
}

template <int D>
static void bwd_outer_d(const BwdArgs &a, int mode, hipStream_t st) {
  const int PP = bwd_outer_parts(a.bh_count, a.nb, mode);
  const dim3 grid(PP, (unsigned)a.bh_count), block(256);
  const dim3 gsum(cdiv(D * 32, 256), (unsigned)a.bh_count), gfin(cdiv(D * 32, 256));
  // the gate-bias partials (k_bwd_dz, run before dS) sit right after the weight partials
  const int64_t bias_at = a.bh_count * 4LL * PP * (D * 32);
  switch (mode) {
    case kOuterRopeQ:
      hipLaunchKernelGGL((k_bwd_outer<D, kOuterRopeQ>), grid, block, 0, st, a, PP);
      hipLaunchKernelGGL((k_bwd_sum<D>), gsum, block, 0, st, a, PP, a.sumtmp);
      hipLaunchKernelGGL((k_bwd_sum_heads<D, false>), gfin, block, 0, st, a, a.sumtmp, bias_at, a.dwq);
      break;
    case kOuterRopeK:
      hipLaunchKernelGGL((k_bwd_outer<D, kOuterRopeK>), grid, block, 0, st, a, PP);
      hipLaunchKernelGGL((k_bwd_sum<D>), gsum, block, 0, st, a, PP, a.sumtmp);
      hipLaunchKernelGGL((k_bwd_sum_heads<D, false>), gfin, block, 0, st, a, a.sumtmp, bias_at, a.dwk);
      break;
    case kOuterDout:
      hipLaunchKernelGGL((k_bwd_outer<D, kOuterDout>), grid, block, 0, st, a, PP);
      hipLaunchKernelGGL((k_bwd_sum<D>), gsum, block, 0, st, a, PP, a.ds32);
      break;
    default:
      hipLaunchKernelGGL((k_bwd_outer<D, kOuterGate>), grid, block, 0, st, a, PP);
      hipLaunchKernelGGL((k_bwd_sum<D>), gsum, block, 0, st, a, PP, a.sumtmp);
      hipLaunchKernelGGL((k_bwd_sum_heads<D, true>), gfin, block, 0, st, a, a.sumtmp, bias_at, a.dgate);
      break;
  }
}

void launch_bwd_outer(const BwdArgs &a, int D, int mode, hipStream_t st) {
  if (D == 64) bwd_outer_d<64>(a, mode, st);
  else bwd_outer_d<128>(a, mode, st);
}

void launch_bwd_dsops(const BwdArgs &a, int D, hipStream_t st) {
  // dz and the per-head gate-bias partials, then the dS operands
  const int PP = bwd_outer_parts(a.bh_count, a.nb, kOuterGate);
  const int64_t bias_at = a.bh_count * 4LL * PP * (D * 32);
  hipLaunchKernelGGL(k_bwd_dz, dim3(kDzParts, (unsigned)a.bh_count), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_bwd_dz2, dim3((unsigned)a.bh_count), dim3(64), 0, st, a, bias_at);
  if (a.comp) return;  // the complement scope's operands are per key block (k_bwd_dsc)
  const dim3 grid(cdiv(a.bh_count * D * 32, 256));
  if (D == 64) hipLaunchKernelGGL(k_bwd_dsops<64>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_dsops<128>, grid, dim3(256), 0, st, a);
}

void launch_bwd_comp_parts(const BwdArgs &a, int D, hipStream_t st) {
  const int PP = cdiv(a.nb, 4);  // one query block per wave
  const dim3 grid(PP, (unsigned)a.bh_count), block(256);
  if (D == 64) hipLaunchKernelGGL((k_bwd_outer<64, kOuterDoutBlk>), grid, block, 0, st, a, PP);
  else hipLaunchKernelGGL((k_bwd_outer<128, kOuterDoutBlk>), grid, block, 0, st, a, PP);
  hipLaunchKernelGGL(k_bwd_dzblk, grid, block, 0, st, a);
  const dim3 gsum(cdiv(D * 32, 256), (unsigned)a.bh_count);
  if (D == 64) hipLaunchKernelGGL(k_bwd_sumblk<64>, gsum, block, 0, st, a);
  else hipLaunchKernelGGL(k_bwd_sumblk<128>, gsum, block, 0, st, a);
}

void launch_bwd_comp_keys(const BwdArgs &a, int D, hipStream_t st) {
  const dim3 grid((unsigned)a.nb, (unsigned)a.bh_count);
  if (D == 64) hipLaunchKernelGGL(k_bwd_dsc<64>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_dsc<128>, grid, dim3(256), 0, st, a);
}

void launch_bwd_key(const BwdArgs &a, int D, hipStream_t st) {
  const dim3 grid(cdiv(2 * a.nb, 4), (unsigned)a.bh_count);
  if (D == 64) hipLaunchKernelGGL(k_bwd_key<64>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_key<128>, grid, dim3(256), 0, st, a);
}

void launch_bwd_dq(const BwdArgs &a, int D, hipStream_t st) {
  // a group's union has at most min(G * kb, nb) entries
  if (a.ugroup && (a.list_stride < a.nb ? a.list_stride : (int64_t)a.nb) <= kDqgLmax && attn_group_size() == 4) {
    // the forward's group schedule: one workgroup of 8 waves per group
    const dim3 grid((unsigned)(8 * a.groups_per_xcd * a.bh_count));
    if (D == 64) hipLaunchKernelGGL((k_bwd_dqg<64, 4>), grid, dim3(512), 0, st, a);
    else hipLaunchKernelGGL((k_bwd_dqg<128, 4>), grid, dim3(512), 0, st, a);
    return;
  }
  const dim3 grid((unsigned)a.nb, (unsigned)a.bh_count);
  if (D == 64) hipLaunchKernelGGL(k_bwd_dq<64>, grid, dim3(128), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_dq<128>, grid, dim3(128), 0, st, a);
}

void launch_bwd_tmap(const BwdArgs &a, hipStream_t st) {
  const size_t lds = (size_t)((a.nb + 31) / 32) * 4;
  hipLaunchKernelGGL(k_bwd_mapbits, dim3((unsigned)a.nb, (unsigned)a.bh_count), dim3(64), lds, st, a);
  hipLaunchKernelGGL(k_bwd_tmap, dim3(cdiv(a.nb, 256), (unsigned)a.bh_count), dim3(256), 0, st, a);
}

void launch_bwd_dkv(const BwdArgs &a, int D, hipStream_t st) {
  const dim3 grid((unsigned)a.nb, (unsigned)a.bh_count);
  if (D == 64) hipLaunchKernelGGL(k_bwd_dkv<64>, grid, dim3(128), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_dkv<128>, grid, dim3(128), 0, st, a);
}

}  // namespace rola
