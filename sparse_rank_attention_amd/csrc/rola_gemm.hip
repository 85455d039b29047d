// rola_gemm.hip -- the w8a8 linear layers either side of attention in the
// fp8 pipeline (README "AlibabaResearch/SparkDiffusion", highlights: optional
// weight-activation quantisation; project page, section "FP8 Quantization &
// Fused Kernels"): per-row e4m3 quantisation of activations (per token) and
// weights (per output channel), and the scaled fp8 product
//   y[m, n] = sx[m] * sw[n] * sum_k value(x[m, k]) * value(w[n, k]) + bias[n]
// on v_mfma_f32_32x32x64_f8f6f4 with fp32 accumulation.
#include "rola_device.h"

namespace rola {

// ------------------------------------------------------ row quantisation
// One wave per row, four rows per 256-thread block.  Row absmax in fp32,
// scale fl32(absmax/448) and inverse fl32(448/absmax) (1 and 1 for a zero
// row), codes RNE-saturated from fl32(x * inverse), eight per lane per step.
// Rows of up to 8192 columns are read once and held in registers; longer
// rows are read twice (the second pass mostly from cache).
constexpr int kQuantRegChunks = 16;

static __device__ __forceinline__ uint2 quant8(u32x4 w, float inv) {
  int lo = cvt_fp8x2<false>(bflo(w[0]) * inv, bfhi(w[0]) * inv, 0);
  lo = cvt_fp8x2<true>(bflo(w[1]) * inv, bfhi(w[1]) * inv, lo);
  int hi = cvt_fp8x2<false>(bflo(w[2]) * inv, bfhi(w[2]) * inv, 0);
  hi = cvt_fp8x2<true>(bflo(w[3]) * inv, bfhi(w[3]) * inv, hi);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

static __device__ __forceinline__ float absmax8(u32x4 w, float m) {
#pragma unroll
  for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bflo(w[j])), fabsf(bfhi(w[j]))));
  return m;
}

static __device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// NCH > 0: the row (at most 512 * NCH columns) is held in NCH chunk
// registers per lane; NCH = 0: two passes over the row
template <int NCH>
__global__ __launch_bounds__(256) void k_quant_rows(QuantRowsArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const uint16_t *xr = a.x + row * a.ldx;
  uint8_t *cr = a.codes + row * a.ldc;
  float m = 0.0f;
  if constexpr (NCH > 0) {
    u32x4 w[NCH];
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
      const int64_t c = (int64_t)lane * 8 + 512 * t;
      w[t] = c < a.cols ? *(const u32x4 *)(xr + c) : u32x4{};
      m = absmax8(w[t], m);
    }
    m = wave_max(m);
    const float inv = m > 0.0f ? __fdiv_rn(448.0f, m) : 1.0f;
    if (lane == 0) a.scale[row] = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
      const int64_t c = (int64_t)lane * 8 + 512 * t;
      if (c < a.cols) *(uint2 *)(cr + c) = quant8(w[t], inv);
    }
  } else {
    for (int64_t c = (int64_t)lane * 8; c < a.cols; c += 512) m = absmax8(*(const u32x4 *)(xr + c), m);
    m = wave_max(m);
    const float inv = m > 0.0f ? __fdiv_rn(448.0f, m) : 1.0f;
    if (lane == 0) a.scale[row] = m > 0.0f ? __fdiv_rn(m, 448.0f) : 1.0f;
    for (int64_t c = (int64_t)lane * 8; c < a.cols; c += 512) *(uint2 *)(cr + c) = quant8(*(const u32x4 *)(xr + c), inv);
  }
}

void launch_quant_rows(const QuantRowsArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
  // the fewest chunk registers that hold the row (fewer registers, more
  // waves in flight)
  const int64_t nch = (a.cols + 511) / 512;
  if (nch <= 2) hipLaunchKernelGGL(k_quant_rows<2>, grid, block, 0, st, a);
  else if (nch <= 4) hipLaunchKernelGGL(k_quant_rows<4>, grid, block, 0, st, a);
  else if (nch <= 6) hipLaunchKernelGGL(k_quant_rows<6>, grid, block, 0, st, a);
  else if (nch <= 8) hipLaunchKernelGGL(k_quant_rows<8>, grid, block, 0, st, a);
  else if (nch <= 10) hipLaunchKernelGGL(k_quant_rows<10>, grid, block, 0, st, a);
  else if (nch <= 12) hipLaunchKernelGGL(k_quant_rows<12>, grid, block, 0, st, a);
  else if (nch <= kQuantRegChunks) hipLaunchKernelGGL(k_quant_rows<kQuantRegChunks>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(k_quant_rows<0>, grid, block, 0, st, a);
}

// ------------------------------------------------------------ fp8 GEMM
// Workgroup tile: 256 output channels x 256 tokens, eight waves (two per
// SIMD, so one wave's MFMAs cover the other's LDS reads and barrier) in a
// 2 x 4 grid of 128 channels x 64 tokens.  The MFMA's A operand is the weight tile (rows =
// channels) and its B operand the activation tile (columns = tokens), so a
// lane's accumulator holds four consecutive channels of one token per
// register quad and stores 8 (bf16) or 16 (fp32) contiguous bytes.
//
// K is staged 64 bytes at a time through a four-slot LDS ring (32 KB per
// slot: 256 weight rows then 256 token rows of 64 bytes) filled by direct
// global->LDS copies issued three stages ahead.  A row's 16-byte chunk c sits at
// chunk position c ^ gemm_swz(row), which makes the operand reads (lane l:
// row l%32, chunks 2g and 2g+1 for lane half g) free of bank conflicts for
// 8-lane (32-bank) and 16-lane (64-bank) service groups alike.
constexpr int kGemmTileT = 256;
constexpr int kGemmTileC = 256;
constexpr int kGemmK = 64;
constexpr int kGemmSlots = 4;
constexpr int kGemmSlotBytes = (kGemmTileT + kGemmTileC) * kGemmK;
constexpr int kGemmGroupM = 4;  // token tiles per group of the tile order

static __device__ __forceinline__ int gemm_swz(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | ((r >> 1) & 2); }

// waves along channels x waves along tokens; each wave owns TI x TJ MFMA
// tiles of 32 x 32
constexpr int kGemmWC = 2, kGemmWT = 4;
// Per-thread copies of a stage: 16 of 1 KB for each part, spread over the waves.
constexpr int kGemmCopies = 32 / (kGemmWC * kGemmWT);

template <int N>
static __device__ __forceinline__ void wait_gemm_stages() {
  wait_vmcnt<N * kGemmCopies>();
}
static __device__ __forceinline__ void wait_gemm_later(int later) {
  if (later >= 3) wait_gemm_stages<3>();
  else if (later == 2) wait_gemm_stages<2>();
  else if (later == 1) wait_gemm_stages<1>();
  else wait_gemm_stages<0>();
}

// workgroup barrier without waiting for this wave's LDS reads (their
// results are awaited where the MFMAs use them)
static __device__ __forceinline__ void barrier_plain() { asm volatile("s_barrier" ::: "memory"); }

static __device__ __forceinline__ i32x8 cat8(u32x4 a, u32x4 b) {
  const u32x4 lo = a, hi = b;
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr int kGemmWaves = kGemmWC * kGemmWT;
constexpr int kGemmTI = kGemmTileC / 32 / kGemmWC, kGemmTJ = kGemmTileT / 32 / kGemmWT;
constexpr int kGemmOps = 16 / kGemmWaves;  // 1 KB copies per wave per part per stage
static_assert(kGemmWaves == 4 || kGemmWaves == 8, "4 or 8 waves");

struct GemmRegs {
  i32x8 w[kGemmTI], x[kGemmTJ];
};

// y = acc * (sx[token] * sw[channel]) + bias[channel] for a wave's TI x TJ
// tiles, stored 4 consecutive channels per lane and register quad
template <bool F32OUT>
static __device__ __forceinline__ void gemm_epilogue(const GemmArgs &a, const f32x16 (&acc)[kGemmTI][kGemmTJ],
                                                     int64_t tok0, int ch0, int wc, int wt, int rl, int g) {
#pragma unroll
  for (int j = 0; j < kGemmTJ; ++j) {
    const int64_t token = tok0 + 32 * kGemmTJ * wt + 32 * j + rl;
    if (token >= a.M) continue;
    const float sxt = a.sx[token];
#pragma unroll
    for (int i = 0; i < kGemmTI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = ch0 + 32 * kGemmTI * wc + 32 * i + 8 * q + 4 * g;
        if (ch >= a.N) continue;
        const f32x4 swv = *(const f32x4 *)(a.sw + ch);
        const f32x4 bv = a.bias ? *(const f32x4 *)(a.bias + ch) : f32x4{};
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fmaf(acc[i][j][4 * q + e], sxt * swv[e], bv[e]);
        if constexpr (F32OUT) {
          *(f32x4 *)((float *)a.out + token * a.ldo + ch) = y;
        } else {
          const __bf16 b0 = (__bf16)y[0], b1 = (__bf16)y[1], b2 = (__bf16)y[2], b3 = (__bf16)y[3];
          const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
          const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
          *(uint2 *)((uint16_t *)a.out + token * a.ldo + ch) = make_uint2(lo, hi);
        }
      }
    }
  }
}

// tile origin of workgroup b: each XCD (workgroups b = x mod 8) takes a
// contiguous range of tiles; within it, groups of kGemmGroupM token tiles
// sweep all channel tiles with the token tile fastest, so the tiles resident
// on one XCD share their activation and weight panels in its L2
static __device__ __forceinline__ void gemm_tile_origin(const GemmArgs &a, int b, int64_t &tok0, int &ch0) {
  const int ntiles = a.tiles_t * a.tiles_c;
  const int per = ntiles / 8, rem = ntiles % 8, xcd = b % 8, idx = b / 8;
  const int t = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
  const int group = t / (kGemmGroupM * a.tiles_c);
  const int first = group * kGemmGroupM;
  const int gm = min(kGemmGroupM, a.tiles_t - first);
  const int within = t - group * kGemmGroupM * a.tiles_c;
  tok0 = (int64_t)(first + within % gm) * kGemmTileT;
  ch0 = (within / gm) * kGemmTileC;
}

template <bool F32OUT>
__global__ __launch_bounds__(64 * kGemmWaves) __attribute__((amdgpu_waves_per_eu(kGemmWaves / 4, kGemmWaves / 4)))
void k_gemm_w8a8(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGemmSlots * kGemmSlotBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;

  int64_t tok0;
  int ch0;
  gemm_tile_origin(a, blockIdx.x, tok0, ch0);

  // copy offsets: op o covers LDS rows 16*(waves*o+wave) .. +16 of each
  // part; rows past the matrix end repeat its last row (never stored)
  uint32_t vw[kGemmOps], vx[kGemmOps];
#pragma unroll
  for (int o = 0; o < kGemmOps; ++o) {
    const int r = 16 * (kGemmWaves * o + wave) + (lane >> 2);
    const int c = (lane & 3) ^ gemm_swz(r);
    const int64_t rw = min((int64_t)ch0 + r, (int64_t)a.N - 1) - ch0;
    const int64_t rx = min(tok0 + r, a.M - 1) - tok0;
    vw[o] = (uint32_t)(rw * a.ldw + 16 * c);
    vx[o] = (uint32_t)(rx * a.ldx + 16 * c);
  }
  const uint8_t *wbase = a.w + (int64_t)ch0 * a.ldw;
  const uint8_t *xbase = a.x + tok0 * a.ldx;
  const uint32_t lds0 = lds_addr(smem);
  const int KT = a.K / kGemmK;

  auto issue = [&](int kt) {
    const uint32_t sb = lds0 + (uint32_t)(kt % kGemmSlots) * kGemmSlotBytes;
    const uint8_t *wb = wbase + (int64_t)kt * kGemmK;
    const uint8_t *xb = xbase + (int64_t)kt * kGemmK;
#pragma unroll
    for (int o = 0; o < kGemmOps; ++o) lds_dma16_m0(wb, vw[o], sb + (uint32_t)(kGemmWaves * o + wave) * 1024);
#pragma unroll
    for (int o = 0; o < kGemmOps; ++o)
      lds_dma16_m0(xb, vx[o], sb + (uint32_t)(kGemmTileC * kGemmK) + (uint32_t)(kGemmWaves * o + wave) * 1024);
  };

  // operand reads: the swizzle depends on row bits 1..3 only, i.e. on lane
  const int wc = wave % kGemmWC, wt = wave / kGemmWC;
  const int rl = lane & 31;
  const uint32_t off0 = (uint32_t)(rl * kGemmK + 16 * ((2 * g) ^ gemm_swz(rl)));
  const uint32_t off1 = (uint32_t)(rl * kGemmK + 16 * ((2 * g + 1) ^ gemm_swz(rl)));
  auto read_w = [&](int slot, int i) -> i32x8 {
    const LDS_AS uint8_t *p = (const LDS_AS uint8_t *)(LDS_AS void *)smem + slot * kGemmSlotBytes +
                              (32 * kGemmTI * wc + 32 * i) * kGemmK;
    return cat8(*(const LDS_AS u32x4 *)(p + off0), *(const LDS_AS u32x4 *)(p + off1));
  };
  auto read_x = [&](int slot, int j) -> i32x8 {
    const LDS_AS uint8_t *p = (const LDS_AS uint8_t *)(LDS_AS void *)smem + slot * kGemmSlotBytes +
                              kGemmTileC * kGemmK + (32 * kGemmTJ * wt + 32 * j) * kGemmK;
    return cat8(*(const LDS_AS u32x4 *)(p + off0), *(const LDS_AS u32x4 *)(p + off1));
  };
  auto read = [&](int slot, GemmRegs &R) {
#pragma unroll
    for (int i = 0; i < kGemmTI; ++i) R.w[i] = read_w(slot, i);
#pragma unroll
    for (int j = 0; j < kGemmTJ; ++j) R.x[j] = read_x(slot, j);
  };

  f32x16 acc[kGemmTI][kGemmTJ];
#pragma unroll
  for (int i = 0; i < kGemmTI; ++i)
#pragma unroll
    for (int j = 0; j < kGemmTJ; ++j) acc[i][j] = f32x16{};

  // stage s is copied into slot s % S during step s - (S-1), read into
  // registers during step s - 1 and multiplied in step s, so the slot a step
  // overwrites was read two steps earlier: its reads are complete (their
  // MFMAs have issued) once every wave has reached the barrier
  constexpr int S = kGemmSlots;
  static_assert(S >= 3 && S <= 5, "LDS ring of 3 to 5 slots");
  const int pre = min(S - 1, KT);
  for (int s = 0; s < pre; ++s) issue(s);
  wait_gemm_later(pre - 1);
  barrier_plain();

  GemmRegs R;
  read(0, R);

  // one stage of MFMAs; with MORE, each operand register is refilled with
  // the next stage (slot sn) right after its last MFMA of this one
  auto stage = [&](auto more_c, int sn) {
    constexpr bool MORE = decltype(more_c)::value;
#pragma unroll
    for (int i = 0; i < kGemmTI; ++i) {
#pragma unroll
      for (int j = 0; j < kGemmTJ; ++j) {
        acc[i][j] = mfma_fp8(R.w[i], R.x[j], acc[i][j]);
        if (MORE && i == kGemmTI - 1) R.x[j] = read_x(sn, j);
      }
      if (MORE) R.w[i] = read_w(sn, i);
    }
    // let each operand read issue between two MFMAs
    if (MORE) {
#pragma unroll
      for (int u = 0; u < kGemmTI * kGemmTJ; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  for (int kt = 0; kt + 1 < KT; ++kt) {
    wait_gemm_later(min(KT - 1, kt + S - 2) - (kt + 1));
    barrier_plain();
    if (kt + S - 1 < KT) issue(kt + S - 1);
    stage(std::true_type{}, (kt + 1) % kGemmSlots);
  }
  stage(std::false_type{}, 0);

  gemm_epilogue<F32OUT>(a, acc, tok0, ch0, wc, wt, rl, g);
}

// The same tile with K staged 128 bytes at a time: two 64 KB slots (256
// weight rows, then 256 token rows, of 128 bytes), each row copied as one
// full 128-byte line by 8 lanes.  Stage kt+1 is copied while stage kt is
// multiplied; a stage's operands are read within its own step (the other
// wave on the SIMD covers the first reads).  Chunk c of row r sits at
// c ^ gemm_swz128(r): free of bank conflicts for rows read 8 or 16 at a time.
constexpr int kGemmK2 = 128;
constexpr int kGemmSlotBytes2 = (kGemmTileT + kGemmTileC) * kGemmK2;
constexpr int kGemmOps2 = 32 / kGemmWaves;  // 1 KB copies per wave per part per stage

static __device__ __forceinline__ int gemm_swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <bool F32OUT>
__global__ __launch_bounds__(64 * kGemmWaves) __attribute__((amdgpu_waves_per_eu(kGemmWaves / 4, kGemmWaves / 4)))
void k_gemm_w8a8_k128(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kGemmSlotBytes2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  int64_t tok0;
  int ch0;
  gemm_tile_origin(a, blockIdx.x, tok0, ch0);

  // copy offsets: op o covers LDS rows 8*(waves*o+wave) .. +8 of each part
  uint32_t vw[kGemmOps2], vx[kGemmOps2];
#pragma unroll
  for (int o = 0; o < kGemmOps2; ++o) {
    const int r = 8 * (kGemmWaves * o + wave) + (lane >> 3);
    const int c = (lane & 7) ^ gemm_swz128(r);
    const int64_t rw = min((int64_t)ch0 + r, (int64_t)a.N - 1) - ch0;
    const int64_t rx = min(tok0 + r, a.M - 1) - tok0;
    vw[o] = (uint32_t)(rw * a.ldw + 16 * c);
    vx[o] = (uint32_t)(rx * a.ldx + 16 * c);
  }
  const uint8_t *wbase = a.w + (int64_t)ch0 * a.ldw;
  const uint8_t *xbase = a.x + tok0 * a.ldx;
  const uint32_t lds0 = lds_addr(smem);
  const int KT = a.K / kGemmK2;
  auto issue = [&](int kt) {
    const uint32_t sb = lds0 + (uint32_t)(kt & 1) * kGemmSlotBytes2;
    const uint8_t *wb = wbase + (int64_t)kt * kGemmK2;
    const uint8_t *xb = xbase + (int64_t)kt * kGemmK2;
#pragma unroll
    for (int o = 0; o < kGemmOps2; ++o) lds_dma16_m0(wb, vw[o], sb + (uint32_t)(kGemmWaves * o + wave) * 1024);
#pragma unroll
    for (int o = 0; o < kGemmOps2; ++o)
      lds_dma16_m0(xb, vx[o], sb + (uint32_t)(kGemmTileC * kGemmK2) + (uint32_t)(kGemmWaves * o + wave) * 1024);
  };

  const int wc = wave % kGemmWC, wt = wave / kGemmWC;
  const int rl = lane & 31;
  // operand of k-step ks (0, 1) of a stage: chunks 4ks + 2g and 4ks + 2g + 1
  auto rd = [&](int slot, int row0, int ks) -> i32x8 {
    const LDS_AS uint8_t *p = (const LDS_AS uint8_t *)(LDS_AS void *)smem + slot * kGemmSlotBytes2 +
                              (row0 + rl) * kGemmK2;
    const int sw = gemm_swz128(rl);
    return cat8(*(const LDS_AS u32x4 *)(p + 16 * ((4 * ks + 2 * g) ^ sw)),
                *(const LDS_AS u32x4 *)(p + 16 * ((4 * ks + 2 * g + 1) ^ sw)));
  };
  auto read_w = [&](int slot, int i, int ks) { return rd(slot, 32 * kGemmTI * wc + 32 * i, ks); };
  auto read_x = [&](int slot, int j, int ks) { return rd(slot, kGemmTileC + 32 * kGemmTJ * wt + 32 * j, ks); };

  f32x16 acc[kGemmTI][kGemmTJ];
#pragma unroll
  for (int i = 0; i < kGemmTI; ++i)
#pragma unroll
    for (int j = 0; j < kGemmTJ; ++j) acc[i][j] = f32x16{};

  issue(0);
  GemmRegs R;
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmcnt<0>();  // this wave's copies of stage kt
    barrier_plain();  // every wave's copies landed; slot (kt+1)&1 (stage kt-1) fully read
    if (kt + 1 < KT) issue(kt + 1);
    const int sl = kt & 1;
    // in the order the first MFMAs need them: the first one waits for two reads
    R.w[0] = read_w(sl, 0, 0);
#pragma unroll
    for (int j = 0; j < kGemmTJ; ++j) R.x[j] = read_x(sl, j, 0);
#pragma unroll
    for (int i = 1; i < kGemmTI; ++i) R.w[i] = read_w(sl, i, 0);
    // k-step 0, refilling each operand with k-step 1 after its last MFMA
#pragma unroll
    for (int i = 0; i < kGemmTI; ++i) {
#pragma unroll
      for (int j = 0; j < kGemmTJ; ++j) {
        acc[i][j] = mfma_fp8(R.w[i], R.x[j], acc[i][j]);
        if (i == kGemmTI - 1) R.x[j] = read_x(sl, j, 1);
      }
      R.w[i] = read_w(sl, i, 1);
    }
#pragma unroll
    for (int u = 0; u < kGemmTI * kGemmTJ; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < kGemmTI; ++i)
#pragma unroll
      for (int j = 0; j < kGemmTJ; ++j) acc[i][j] = mfma_fp8(R.w[i], R.x[j], acc[i][j]);
  }
  gemm_epilogue<F32OUT>(a, acc, tok0, ch0, wc, wt, rl, g);
}

// K a multiple of 128 takes the 128-byte stages (4 % faster at 75600 x 5120
// x 15360 than 64-byte stages), otherwise the 64-byte ring

void launch_gemm_w8a8(const GemmArgs &a, hipStream_t st) {
  const int ntiles = a.tiles_t * a.tiles_c;
  if (a.K % kGemmK2 == 0) {
    if (a.out_f32)
      hipLaunchKernelGGL(k_gemm_w8a8_k128<true>, dim3((unsigned)ntiles), dim3(64 * kGemmWaves), 0, st, a);
    else
      hipLaunchKernelGGL(k_gemm_w8a8_k128<false>, dim3((unsigned)ntiles), dim3(64 * kGemmWaves), 0, st, a);
    return;
  }
  if (a.out_f32)
    hipLaunchKernelGGL(k_gemm_w8a8<true>, dim3((unsigned)ntiles), dim3(64 * kGemmWaves), 0, st, a);
  else
    hipLaunchKernelGGL(k_gemm_w8a8<false>, dim3((unsigned)ntiles), dim3(64 * kGemmWaves), 0, st, a);
}

}  // namespace rola
